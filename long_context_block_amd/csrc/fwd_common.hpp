// fwd_common.hpp — device helpers shared by the bf16 forward kernels (gfx950).
#pragma once

#include "bsa_internal.hpp"

namespace bsa {
namespace fwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kRescaleSlack = 8.0f;  // log2 units: P values stay <= 2^8 between rescales
constexpr int KC = 64;                 // keys per LDS chunk (one asynchronous copy unit)
constexpr float kLn2 = 0.69314718055994530942f;

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1))
__device__ inline float dot2_bf16_ones(uint32_t packed, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

// LDS layouts of a K or V chunk: row-major [key][d] with 16-byte chunks XOR-swizzled per row.
//  K: chunk c of row r at c ^ kswz(r): the S^T operand reads (32 consecutive rows, one chunk
//     per half-wavefront) hit distinct banks.
//  V: chunk c of row r at c ^ vswz(r): the transposing reads (4 consecutive rows x 32 columns
//     per half-wavefront) hit distinct banks.
template <int D>
struct Swz {
    static constexpr int KCH = D / 8;  // 16-byte chunks per row
    __device__ static inline int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static inline int vswz(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
    __device__ static inline int k_off(int r, int c) { return r * D + ((c ^ kswz(r)) << 3); }
    __device__ static inline int v_off(int r, int col) { return r * D + (((col >> 3) ^ vswz(r)) << 3) + (col & 7); }
};

// A-operand fragment of V^T for MFMA 32x32x16 (rows d = 32db + lane%32, keys k0 + logical 8hf..+8
// in the order of the S^T accumulator layout), read transposed from a row-major V stage with two
// ds_read_b64_tr_b16: each 16-lane group reads a 4-key x 16-column block and the LDS unit hands
// every lane one column of it.
template <int D>
__device__ inline bf16x8 v_fragment(const __bf16* Vs, int vrow, int vcol) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + Swz<D>::v_off(vrow, vcol)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + Swz<D>::v_off(vrow + 8, vcol)));
    const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
}

// The same fragment read at a precomputed element address p of the first row (rows p and
// p + 8 rows).
template <int D>
__device__ inline bf16x8 v_fragment_at(const __bf16* p) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * D));
    const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
}

// Work item k of work-group w in a persistent launch of G work-groups over `total` items
// (head slices of nqb query blocks each).  Items are taken longest row first (largest i) within
// a slice.  Work-groups are dispatched round-robin over the 8 XCDs, so when both counts allow it
// the items are split into 8 contiguous ranges, one per XCD, and the work-groups of an XCD share
// K/V tiles of the same heads in its L2; within a range, work-group c of C takes items in
// serpentine order (c, 2C-1-c, 2C+c, ...), which evens out the row lengths.  Returns false
// past the work-group's last item.
__device__ inline bool work_item(int w, int G, int k, int total, int nqb, int& slice, int& i) {
    const bool xcd = (total % 8 == 0) && (G % 8 == 0);
    const int c = xcd ? w / 8 : w;
    const int C = xcd ? G / 8 : G;
    const int range = xcd ? total / 8 : total;
    const int64_t pos = (int64_t)k * C + ((k & 1) ? C - 1 - c : c);
    if (pos >= range) return false;
    const int vi = (xcd ? (w % 8) * range : 0) + (int)pos;
    slice = vi / nqb;
    i = nqb - 1 - (vi % nqb);
    return true;
}

}  // namespace fwd
}  // namespace bsa

namespace bsa {
namespace fwd {

// Asynchronous copy of 16 bytes per lane from global memory to LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4).  Issued from inline asm so that the compiler does not treat the
// LDS write as aliasing every later LDS read (it would otherwise wait for the copy to land
// before the first operand read of the current stage); completion is awaited explicitly with
// s_waitcnt vmcnt(0) before the barrier that publishes a stage.  lds_base is made
// wavefront-uniform; M0 carries it.  M0 is reserved by the compiler and cannot be declared
// clobbered; the kernels that use this helper contain no other M0 user (build.py checks the
// generated code for that).
__device__ inline void copy16_to_lds(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(src)
                 : "memory");
}

__device__ inline uint32_t lds_addr(const __bf16* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

// The same copy with a wavefront-uniform global base (scalar registers) and a per-lane 32-bit
// byte offset: global_load_lds_dwordx4 in its scalar-base form, so a lane holds one offset
// register instead of a 64-bit address.
__device__ inline void copy16_to_lds(const void* base, uint32_t off, uint32_t lds_base) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    // readfirstlane works on (signed) int: widen each half as unsigned, never sign-extended
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t bu = (hi << 32) | lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(off), "s"(bu)
                 : "memory");
}

}  // namespace fwd
}  // namespace bsa
