// bwd_bf16.hip — gradients of bfloat16 block-sparse attention on gfx950 matrix cores.
//
// What it computes (the "gradients" correctness gate of "BF1 ...", section 4): for the forward
// O = P V, P = softmax(S) over the selected keys, S = scale Q K^T (masked before the softmax:
// "Block-Sparse Attention", "Math Or Compute Schema"), and an upstream gradient dO,
//     dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  D = rowsum(dO * O),
//     dQ = scale dS K,  dK = scale dS^T Q,
// with dK, dV summed over the query heads that share a key/value head.  P is recomputed from Q,
// K and the forward's log-sum-exp; excluded pairs have P = 0 and carry no gradient.
//
// How (gfx950; the structure of the unpipelined forward kernel, run twice):
//  * bwd_prep_kernel: D[t] = sum_d dO[t, d] O[t, d] in fp32, one 16-byte slice per lane.
//  * bwd_dq_kernel: one work-group per (batch, query head, query block i), 32 query rows per
//    wavefront, walking row i of the route in 64-key chunks copied HBM -> LDS one chunk ahead
//    (global_load_lds_dwordx4, two stages).  Per chunk, on the matrix cores: S^T = K Q^T and
//    dP^T = V dO^T (K, V rows from LDS; Q, dO resident in registers), then dS^T = P^T (dP^T - D)
//    in registers (one query per lane), then dQ^T += K^T dS^T with K^T read transposed by the
//    LDS unit (ds_read_b64_tr_b16).
//  * bwd_dkdv_kernel: the same with the roles of queries and keys exchanged: one work-group per
//    (batch, key/value head, key block j, segment), 32 keys per wavefront (K, V resident in
//    registers), walking the transposed route (the query blocks whose rows hold j) times the
//    query heads of the group, in 64-query chunks of Q and dO (plus their log-sum-exp and D)
//    copied to LDS.  Per chunk: S = Q K^T, dP = dO V^T, P and dS, then dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T and Q^T read transposed.  A key block read by many query blocks
//    (block 0 in BF1 is read by all of them) is split into segments of at most kSeg chunks so
//    that no work-group carries a whole column; each segment writes fp32 partials that
//    bwd_dkdv_reduce_kernel sums in segment order (deterministic, no atomics).
//  * Tiles read both row-wise and transposed use one XOR swizzle of 16-byte chunks for both.

#include "fwd_common.hpp"

namespace bsa {
namespace {

using namespace fwd;

constexpr int kCh = 64;     // keys (dq) or queries (dkdv) per LDS chunk
constexpr int kSeg = 64;    // chunks per dkdv segment
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

// Copy rows [row0, row0 + kCh) of a [rows, D] bf16 matrix (rows clamped to last) into an LDS
// tile with the Sw2 swizzle; instruction q of the work-group writes LDS bytes [1024 q, +1024).
template <int D, int NW>
__device__ inline void issue_tile(const __bf16* M, int64_t row0, int64_t last, __bf16* tile, int wv, int lane) {
    constexpr int NI = kCh * D / 512;
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

// Copy kCh floats v[row0 .. row0 + kCh) (indices clamped to last) into LDS, one dword per lane
// of wavefront 0 (global_load_lds_dword).
__device__ inline void issue_vec(const float* v, int64_t row0, int64_t last, float* dst, int wv, int lane) {
    if (wv != 0) return;
    int64_t r = row0 + lane;
    r = r < last ? r : last;
    const uint32_t lb = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)dst;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lb)),
                 "v"(v + r)
                 : "memory");
}

// ---- D = rowsum(dO * O) -------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
    constexpr int LPR = D / 8;  // lanes per row (16 bytes each)
    const int64_t rows = (int64_t)p.batch * p.heads_q * p.n;
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
    const int c = threadIdx.x % LPR;
    float s = 0.f;
    if (row < rows) {
        const uint4 a = *(const uint4*)((const __bf16*)p.d_o + row * D + c * 8);
        const uint4 o = *(const uint4*)((const __bf16*)p.o + row * D + c * 8);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            s = fmaf(__uint_as_float(aw[x] << 16), __uint_as_float(ow[x] << 16), s);
            s = fmaf(__uint_as_float(aw[x] & 0xffff0000u), __uint_as_float(ow[x] & 0xffff0000u), s);
        }
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
    if (row < rows && c == 0) p.dvec[row] = s;
}

// ---- dQ --------------------------------------------------------------------------------------
template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdParams p) {
    constexpr int NW = BLK / 32;
    constexpr int CPB = BLK / kCh;  // chunks per key block
    __shared__ __attribute__((aligned(1024))) __bf16 sK[2][kCh * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV[2][kCh * D];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hf = lane >> 5;
    const int64_t total = (int64_t)p.batch * p.heads_q * p.nqb;
    const int64_t w = blockIdx.x;
    const int64_t vi = (total % 8 == 0) ? (w % 8) * (total / 8) + w / 8 : w;  // XCD-contiguous slices
    const int64_t bh = vi / p.nqb;                       // batch * heads_q + h
    const int64_t i = p.nqb - 1 - (vi % p.nqb);          // longest rows first
    const int64_t b = bh / p.heads_q, h = bh % p.heads_q;
    const int64_t kvh = h / (p.heads_q / p.heads_kv);
    const int64_t n = p.n;
    const __bf16* Kg = (const __bf16*)p.k + (b * p.heads_kv + kvh) * n * D;
    const __bf16* Vg = (const __bf16*)p.v + (b * p.heads_kv + kvh) * n * D;

    const int qloc = 32 * wv + l32;
    const int64_t qrow = i * BLK + qloc;
    const bool row_ok = qrow < n;
    bf16x8 qf[D / 16], dof[D / 16];
    {
        const __bf16* Qr = (const __bf16*)p.q + (bh * n + (row_ok ? qrow : 0)) * D;
        const __bf16* Gr = (const __bf16*)p.d_o + (bh * n + (row_ok ? qrow : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            qf[kk] = row_ok ? *(const bf16x8*)(Qr + 16 * kk + 8 * hf) : bf16x8{};
            dof[kk] = row_ok ? *(const bf16x8*)(Gr + 16 * kk + 8 * hf) : bf16x8{};
        }
    }
    const float lse2 = row_ok ? p.lse[bh * n + qrow] * kLog2e : 0.f;
    const float dval = row_ok ? p.dvec[bh * n + qrow] : 0.f;

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    int64_t e0 = p.row_ptr[i], e1 = p.row_ptr[i + 1];
    e0 = e0 < 0 ? 0 : (e0 > p.nnz ? p.nnz : e0);
    e1 = e1 < e0 ? e0 : (e1 > p.nnz ? p.nnz : e1);
    const int NCH = (int)(e1 - e0) * CPB;
    const cptr cidx = (cptr)p.col_idx;
    auto block_of = [&](int ch) -> int64_t {
        const int64_t j = __builtin_amdgcn_readfirstlane(cidx[e0 + ch / CPB]);
        return (j < 0 || j > i) ? -1 : j;
    };
    auto issue = [&](int ch, int st) {
        const int64_t j = block_of(ch);
        const int64_t row0 = (j >= 0 ? j : i) * BLK + kCh * (ch % CPB);
        issue_tile<D, NW>(Kg, row0, n - 1, sK[st], wv, lane);
        issue_tile<D, NW>(Vg, row0, n - 1, sV[st], wv, lane);
    };
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    if (NCH > 0) issue(0, 0);
    for (int ch = 0; ch < NCH; ++ch) {
        const int st = ch & 1;
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (ch + 1 < NCH) issue(ch + 1, st ^ 1);
        const int64_t j = block_of(ch);
        const int kb = kCh * (ch % CPB);  // first key of the chunk within its block
        // S^T and dP^T for the chunk's 64 keys (two 32-key accumulators each)
        f32x16 s[2], dp[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            s[c2] = f32x16{};
            dp[c2] = f32x16{};
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                s[c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_fragment<D>(sK[st], 32 * c2 + l32, 2 * kk + hf),
                                                                qf[kk], s[c2], 0, 0, 0);
                dp[c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_fragment<D>(sV[st], 32 * c2 + l32, 2 * kk + hf),
                                                                 dof[kk], dp[c2], 0, 0, 0);
            }
        // dS^T = P^T (dP^T - D), packed to bf16; masked pairs (future keys on the diagonal block,
        // malformed entries, rows past n) have P = 0
        const bool diag = (j == i);
        const int lim = (j < 0 || !row_ok) ? -1 : (diag ? qloc - kb : kCh);
        uint32_t pk[2][8];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                float ds[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * x + e;
                    const int key = 32 * c2 + 8 * (r >> 2) + 4 * hf + (r & 3);
                    const float pw = key > lim ? 0.f : __builtin_amdgcn_exp2f(fmaf(s[c2][r], p.scale_log2, -lse2));
                    ds[e] = pw * (dp[c2][r] - dval);
                }
                pk[c2][x] = pack_bf16x2(ds[0], ds[1]);
            }
        // dQ^T[d][q] += K^T[d][k] dS^T[k][q]
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const bf16x8 bop = __builtin_bit_cast(
                    bf16x8, make_uint4(pk[c2][4 * sl], pk[c2][4 * sl + 1], pk[c2][4 * sl + 2], pk[c2][4 * sl + 3]));
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 a = t_fragment<D>(sK[st], 32 * c2 + 16 * sl + vr_lane, 32 * db + vc_lane);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[db], 0, 0, 0);
                }
            }
    }

    if (row_ok) {
        __bf16* Dq = (__bf16*)p.dq + (bh * n + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int d0 = 32 * db + 8 * j4 + 4 * hf;
                const uint32_t w0 = pack_bf16x2(acc[db][4 * j4] * p.scale, acc[db][4 * j4 + 1] * p.scale);
                const uint32_t w1 = pack_bf16x2(acc[db][4 * j4 + 2] * p.scale, acc[db][4 * j4 + 3] * p.scale);
                *(uint2*)(Dq + d0) = make_uint2(w0, w1);
            }
    }
}

// ---- segments of the transposed route ----------------------------------------------------------
// seg_ptr[j] = sum over j' < j of max(1, ceil(chunks(j') / kSeg)), chunks(j) = |RT(j)| * G * BLK/kCh
__global__ __launch_bounds__(1024) void bwd_seg_kernel(BwdParams p, int cpb) {
    __shared__ int64_t part[1024];
    const int t = threadIdx.x;
    const int64_t nqb = p.nqb;
    const int G = p.heads_q / p.heads_kv;
    const int64_t per = (nqb + 1023) / 1024;
    const int64_t r0 = t * per, r1 = (r0 + per < nqb) ? r0 + per : nqb;
    auto segs = [&](int64_t j) -> int64_t {
        int64_t a = p.t_row_ptr[j], z = p.t_row_ptr[j + 1];
        a = a < 0 ? 0 : (a > p.nnz ? p.nnz : a);
        z = z < a ? a : (z > p.nnz ? p.nnz : z);
        const int64_t len = z - a;
        const int64_t c = len * G * cpb;
        const int64_t s = (c + kSeg - 1) / kSeg;
        return s > 1 ? s : 1;
    };
    int64_t local = 0;
    for (int64_t j = r0; j < r1; ++j) local += segs(j);
    part[t] = local;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int64_t add = (t >= off) ? part[t - off] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    int64_t run = part[t] - local;
    for (int64_t j = r0; j < r1; ++j) {
        p.seg_ptr[j] = (int32_t)run;
        run += segs(j);
    }
    if (t == 1023) p.seg_ptr[nqb] = (int32_t)part[1023];
}

// ---- dK, dV ----------------------------------------------------------------------------------
template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(BwdParams p) {
    constexpr int NW = BLK / 32;
    constexpr int CPB = BLK / kCh;  // chunks per query block
    __shared__ __attribute__((aligned(1024))) __bf16 sQ[2][kCh * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sO[2][kCh * D];  // dO
    __shared__ __attribute__((aligned(16))) float sL[2][kCh];
    __shared__ __attribute__((aligned(16))) float sD[2][kCh];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, hf = lane >> 5;
    const int64_t bg = blockIdx.x / p.nseg_ub;  // batch * heads_kv + g
    const int sw = (int)(blockIdx.x % p.nseg_ub);
    const int64_t nqb = p.nqb;
    if (sw >= p.seg_ptr[nqb]) return;
    // key block j: seg_ptr[j] <= sw < seg_ptr[j + 1]
    int64_t lo = 0, hi = nqb - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (p.seg_ptr[mid] <= sw) lo = mid; else hi = mid - 1;
    }
    const int64_t j = lo;
    const int seg = sw - p.seg_ptr[j];
    const int nseg = p.seg_ptr[j + 1] - p.seg_ptr[j];
    const int64_t b = bg / p.heads_kv, g = bg % p.heads_kv;
    const int G = p.heads_q / p.heads_kv;
    const int64_t n = p.n;

    int64_t t0 = p.t_row_ptr[j], t1 = p.t_row_ptr[j + 1];
    t0 = t0 < 0 ? 0 : (t0 > p.nnz ? p.nnz : t0);
    t1 = t1 < t0 ? t0 : (t1 > p.nnz ? p.nnz : t1);
    const int nch_all = (int)(t1 - t0) * G * CPB;
    const int c_begin = seg * kSeg;
    const int c_end = (c_begin + kSeg < nch_all) ? c_begin + kSeg : nch_all;
    const int NCH = c_end > c_begin ? c_end - c_begin : 0;

    // this wavefront's 32 keys, resident as B operands: K[key][16kk + 8hf ..], V likewise
    const int kloc = 32 * wv + l32;
    const int64_t krow = j * BLK + kloc;
    const bool key_ok = krow < n;
    bf16x8 kf[D / 16], vf[D / 16];
    {
        const __bf16* Kr = (const __bf16*)p.k + (bg * n + (key_ok ? krow : 0)) * D;
        const __bf16* Vr = (const __bf16*)p.v + (bg * n + (key_ok ? krow : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            kf[kk] = key_ok ? *(const bf16x8*)(Kr + 16 * kk + 8 * hf) : bf16x8{};
            vf[kk] = key_ok ? *(const bf16x8*)(Vr + 16 * kk + 8 * hf) : bf16x8{};
        }
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    // chunk c -> (query block i, query head h, first query row)
    auto chunk = [&](int c, int64_t& i, int64_t& bh, int64_t& q0) {
        const int ti = c / (G * CPB), rem = c % (G * CPB);
        const int64_t iq = __builtin_amdgcn_readfirstlane(((cptr)p.t_col_idx)[t0 + ti]);
        i = (iq < j || iq >= nqb) ? -1 : iq;  // malformed: a fully masked chunk
        bh = b * p.heads_q + g * G + rem / CPB;
        q0 = (i >= 0 ? i : j) * BLK + kCh * (rem % CPB);
    };
    auto issue = [&](int c, int st) {
        int64_t i, bh, q0;
        chunk(c, i, bh, q0);
        issue_tile<D, NW>((const __bf16*)p.q + bh * n * D, q0, n - 1, sQ[st], wv, lane);
        issue_tile<D, NW>((const __bf16*)p.d_o + bh * n * D, q0, n - 1, sO[st], wv, lane);
        issue_vec(p.lse + bh * n, q0, n - 1, sL[st], wv, lane);
        issue_vec(p.dvec + bh * n, q0, n - 1, sD[st], wv, lane);
    };
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    if (NCH > 0) issue(c_begin, 0);
    for (int cc = 0; cc < NCH; ++cc) {
        const int st = cc & 1;
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (cc + 1 < NCH) issue(c_begin + cc + 1, st ^ 1);
        int64_t i, bh, q0;
        chunk(c_begin + cc, i, bh, q0);
        // S[q][k] and dP[q][k] for the chunk's 64 queries (two 32-query accumulators)
        f32x16 s[2], dp[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            s[c2] = f32x16{};
            dp[c2] = f32x16{};
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                s[c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_fragment<D>(sQ[st], 32 * c2 + l32, 2 * kk + hf),
                                                                kf[kk], s[c2], 0, 0, 0);
                dp[c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_fragment<D>(sO[st], 32 * c2 + l32, 2 * kk + hf),
                                                                 vf[kk], dp[c2], 0, 0, 0);
            }
        // P and dS; a pair is masked when the query precedes the key on the diagonal block, the
        // query row is past n, or the chunk is a malformed entry
        const int64_t qbase = q0 - (i >= 0 ? i : j) * BLK;  // first query of the chunk within its block
        uint32_t pp[2][8], ps[2][8];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int qr = 32 * c2 + 8 * r4 + 4 * hf;  // 4 consecutive query rows of the chunk
                const float4 lq = *(const float4*)&sL[st][qr];
                const float4 dq = *(const float4*)&sD[st][qr];
                const float lv[4] = {lq.x, lq.y, lq.z, lq.w}, dvv[4] = {dq.x, dq.y, dq.z, dq.w};
                float pw[4], dsv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * r4 + e;
                    const int64_t qglob = q0 + qr + e;
                    const bool ok = i >= 0 && qglob < n && !(i == j && qbase + qr + e < kloc);
                    pw[e] = ok ? __builtin_amdgcn_exp2f(fmaf(s[c2][r], p.scale_log2, -lv[e] * kLog2e)) : 0.f;
                    dsv[e] = pw[e] * (dp[c2][r] - dvv[e]);
                }
                pp[c2][2 * r4] = pack_bf16x2(pw[0], pw[1]);
                pp[c2][2 * r4 + 1] = pack_bf16x2(pw[2], pw[3]);
                ps[c2][2 * r4] = pack_bf16x2(dsv[0], dsv[1]);
                ps[c2][2 * r4 + 1] = pack_bf16x2(dsv[2], dsv[3]);
            }
        // dV^T[d][k] += dO^T[d][q] P[q][k];  dK^T[d][k] += Q^T[d][q] dS[q][k]
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const bf16x8 bp = __builtin_bit_cast(
                    bf16x8, make_uint4(pp[c2][4 * sl], pp[c2][4 * sl + 1], pp[c2][4 * sl + 2], pp[c2][4 * sl + 3]));
                const bf16x8 bs = __builtin_bit_cast(
                    bf16x8, make_uint4(ps[c2][4 * sl], ps[c2][4 * sl + 1], ps[c2][4 * sl + 2], ps[c2][4 * sl + 3]));
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const int tr = 32 * c2 + 16 * sl + vr_lane, tc = 32 * db + vc_lane;
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t_fragment<D>(sO[st], tr, tc), bp, dv[db], 0, 0, 0);
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t_fragment<D>(sQ[st], tr, tc), bs, dk[db], 0, 0, 0);
                }
            }
    }

    // lane holds d = 32 db + 8 j4 + 4 hf + (0..3) of key kloc
    if (nseg == 1) {
        if (key_ok) {
            __bf16* Dk = (__bf16*)p.dk + (bg * n + krow) * D;
            __bf16* Dv = (__bf16*)p.dv + (bg * n + krow) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const int d0 = 32 * db + 8 * j4 + 4 * hf;
                    *(uint2*)(Dk + d0) = make_uint2(pack_bf16x2(dk[db][4 * j4] * p.scale, dk[db][4 * j4 + 1] * p.scale),
                                                    pack_bf16x2(dk[db][4 * j4 + 2] * p.scale, dk[db][4 * j4 + 3] * p.scale));
                    *(uint2*)(Dv + d0) = make_uint2(pack_bf16x2(dv[db][4 * j4], dv[db][4 * j4 + 1]),
                                                    pack_bf16x2(dv[db][4 * j4 + 2], dv[db][4 * j4 + 3]));
                }
        }
    } else {
        float* part = p.part + ((int64_t)blockIdx.x * 2) * BLK * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int d0 = 32 * db + 8 * j4 + 4 * hf;
                *(float4*)(part + kloc * D + d0) = make_float4(dk[db][4 * j4], dk[db][4 * j4 + 1], dk[db][4 * j4 + 2],
                                                               dk[db][4 * j4 + 3]);
                *(float4*)(part + (BLK + kloc) * D + d0) = make_float4(dv[db][4 * j4], dv[db][4 * j4 + 1],
                                                                       dv[db][4 * j4 + 2], dv[db][4 * j4 + 3]);
            }
    }
}

// Sum the segments of key blocks split over several work-groups, in segment order.  Work-group
// (b, kv head, j, part) takes 1024 consecutive elements of the block's dK and dV (one float4 of
// each per thread); the segment loop is unrolled so that its loads are in flight together.
constexpr int kRedElems = 1024;
template <int D, int BLK>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(BwdParams p) {
    constexpr int PARTS = BLK * D / kRedElems;
    const int64_t w = blockIdx.x;
    const int part = (int)(w % PARTS);
    const int64_t j = (w / PARTS) % p.nqb;
    const int64_t bg = w / PARTS / p.nqb;
    // (clamped to the workspace's segment slots, so that even a malformed route stays in bounds)
    const int s1 = p.seg_ptr[j + 1] < p.nseg_ub ? p.seg_ptr[j + 1] : (int)p.nseg_ub;
    const int s0 = p.seg_ptr[j] < s1 ? p.seg_ptr[j] : s1;
    if (s1 - s0 < 2) return;
    const int64_t n = p.n;
    const int e = part * kRedElems + threadIdx.x * 4;
    const int r = e / D, c = e % D;
    const int64_t krow = j * BLK + r;
    if (krow >= n) return;
    const float* base = p.part + (bg * p.nseg_ub) * 2 * BLK * D + e;
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    constexpr int U = 8;
    for (int s = s0; s < s1; s += U) {
        float4 a[U], v[U];
#pragma unroll
        for (int x = 0; x < U; ++x) {
            const int sg = s + x < s1 ? s + x : s1 - 1;
            a[x] = *(const float4*)(base + (int64_t)sg * 2 * BLK * D);
            v[x] = *(const float4*)(base + (int64_t)sg * 2 * BLK * D + BLK * D);
        }
#pragma unroll
        for (int x = 0; x < U; ++x) {
            if (s + x < s1) {
                sk.x += a[x].x; sk.y += a[x].y; sk.z += a[x].z; sk.w += a[x].w;
                sv.x += v[x].x; sv.y += v[x].y; sv.z += v[x].z; sv.w += v[x].w;
            }
        }
    }
    __bf16* Dk = (__bf16*)p.dk + (bg * n + krow) * D + c;
    __bf16* Dv = (__bf16*)p.dv + (bg * n + krow) * D + c;
    *(uint2*)Dk = make_uint2(pack_bf16x2(sk.x * p.scale, sk.y * p.scale), pack_bf16x2(sk.z * p.scale, sk.w * p.scale));
    *(uint2*)Dv = make_uint2(pack_bf16x2(sv.x, sv.y), pack_bf16x2(sv.z, sv.w));
}

template <int D, int BLK>
hipError_t launch_t(const BwdParams& p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.batch * p.heads_q * p.n;
    const int64_t prep_blocks = (rows * (D / 8) + 255) / 256;
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)prep_blocks), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_seg_kernel, dim3(1), dim3(1024), 0, stream, p, BLK / kCh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, BLK>), dim3((unsigned)((int64_t)p.batch * p.heads_q * p.nqb)),
                       dim3(BLK / 32 * 64), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, BLK>), dim3((unsigned)((int64_t)p.batch * p.heads_kv * p.nseg_ub)),
                       dim3(BLK / 32 * 64), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<D, BLK>),
                       dim3((unsigned)((int64_t)p.batch * p.heads_kv * p.nqb * (BLK * D / kRedElems))), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

int64_t bwd_segments_upper_bound(int64_t nqb, int64_t nnz, int heads_q, int heads_kv, int block) {
    const int64_t chunks = nnz * (heads_q / heads_kv) * (block / kCh);
    return nqb + (chunks + kSeg - 1) / kSeg;
}

hipError_t launch_bwd_bf16(const BwdParams& p, int d, int block, hipStream_t stream) {
    if (d == 128) return block == 128 ? launch_t<128, 128>(p, stream) : launch_t<128, 64>(p, stream);
    return block == 128 ? launch_t<64, 128>(p, stream) : launch_t<64, 64>(p, stream);
}

}  // namespace bsa
