// bwd_common.hpp — device helpers shared by the backward kernels (gfx950).
#pragma once

#include "fwd_common.hpp"

namespace bsa {
namespace bwd {

using namespace fwd;

constexpr int kCh = 64;     // keys per dQ chunk; queries per unit of a dK/dV segment
constexpr int kSeg = 64;    // 64-query units per dK/dV segment
constexpr float kLog2e = 1.4426950408889634074f;

// wavefront-uniform route reads go through the scalar data cache (counted by lgkmcnt, so they
// never wait for the asynchronous tile copies counted by vmcnt)
typedef const __attribute__((address_space(4))) int32_t* cptr;

// One swizzle for tiles read row-wise (16-byte A fragments) and transposed (ds_read_b64_tr_b16):
// the 16-byte chunk c of row r sits at chunk c ^ f(r).
template <int D>
struct Sw2 {
    static constexpr int KCH = D / 8;
    __device__ static inline int f(int r) {
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r & 1) << 2) | ((r >> 1) & 3));
    }
    __device__ static inline int off(int r, int c) { return r * D + ((c ^ f(r)) << 3); }
    __device__ static inline int toff(int r, int col) { return r * D + (((col >> 3) ^ f(r)) << 3) + (col & 7); }
};

// A operand (rows 32 of a tile, k = 16 columns) read row-wise: tile row `row`, chunk `c`
template <int D>
__device__ inline bf16x8 row_fragment(const __bf16* T, int row, int c) {
    return *(const bf16x8*)(T + Sw2<D>::off(row, c));
}
// A operand of a transposed tile (rows = columns d of the tile, k = 16 tile rows in the order of
// the MFMA accumulator layout): two transposing reads of 4 rows x 16 columns per 16-lane group
template <int D>
__device__ inline bf16x8 t_fragment(const __bf16* T, int trow, int tcol) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(T + Sw2<D>::toff(trow, tcol)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(T + Sw2<D>::toff(trow + 8, tcol)));
    const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
}

// Copy rows [row0, row0 + ROWS) of a [rows, D] bf16 matrix (rows clamped to last) into an LDS
// tile with the Sw2 swizzle; instruction q of the work-group writes LDS bytes [1024 q, +1024).
template <int D, int NW, int ROWS = kCh>
__device__ inline void issue_tile(const __bf16* M, int64_t row0, int64_t last, __bf16* tile, int wv, int lane) {
    constexpr int NI = ROWS * D / 512;
    constexpr int NI_W = NI / NW;
    static_assert(NI_W * NW == NI, "tile split");
    const int64_t b = row0 < last ? row0 : last;
    const int delta = (int)(row0 - b), lim = (int)(last - b);
    const char* base = (const char*)(M + b * D);
#pragma unroll
    for (int u = 0; u < NI_W; ++u) {
        const int qi = wv * NI_W + u;
        const int P = 64 * qi + lane;
        const int r = P / Sw2<D>::KCH, pc = P % Sw2<D>::KCH;
        const int rr = (r + delta) < lim ? (r + delta) : lim;
        copy16_to_lds(base, (uint32_t)(rr * D * 2 + ((pc ^ Sw2<D>::f(r)) << 4)), lds_addr(tile + qi * 512));
    }
}

// The same copy into the LDS byte address `lds` (wavefront-uniform) of the tile.
template <int D, int NW, int ROWS>
__device__ inline void issue_tile_at(const __bf16* M, int64_t row0, int64_t last, uint32_t lds, int wv, int lane) {
    constexpr int NI = ROWS * D / 512;
    constexpr int NI_W = NI / NW;
    static_assert(NI_W * NW == NI, "tile split");
    const int64_t b = row0 < last ? row0 : last;
    const int delta = (int)(row0 - b), lim = (int)(last - b);
    const char* base = (const char*)(M + b * D);
#pragma unroll
    for (int u = 0; u < NI_W; ++u) {
        const int qi = wv * NI_W + u;
        const int P = 64 * qi + lane;
        const int r = P / Sw2<D>::KCH, pc = P % Sw2<D>::KCH;
        const int rr = (r + delta) < lim ? (r + delta) : lim;
        copy16_to_lds(base, (uint32_t)(rr * D * 2 + ((pc ^ Sw2<D>::f(r)) << 4)), lds + 1024u * qi);
    }
}

// One dword per lane of wavefront 0 into LDS: dword `lane` at LDS byte address lds = *src
// (global_load_lds_dword).
__device__ inline void issue_dword_at(const float* src, uint32_t lds, int wv) {
    if (wv != 0) return;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                 "v"(src)
                 : "memory");
}
__device__ inline void issue_dword(const float* src, float* dst, int wv) {
    issue_dword_at(src, (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)dst, wv);
}

// Copy kCh floats v[row0 .. row0 + kCh) (indices clamped to last) into LDS.
__device__ inline void issue_vec(const float* v, int64_t row0, int64_t last, float* dst, int wv, int lane) {
    int64_t r = row0 + lane;
    r = r < last ? r : last;
    issue_dword(v + r, dst, wv);
}

}  // namespace bwd

// dK, dV of the backward (bwd_dkdv.hip): the segment kernel and the ordered segment reduction
// run after seg_ptr is filled; the partials go to p.part.
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, int block, hipStream_t stream);

}  // namespace bsa
