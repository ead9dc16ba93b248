// bsbr.hip — BSBR attention on gfx950: the within-chunk term and the between-chunk retrieval.
//
// What it computes ("bsbr", Solution: the combined formula), per batch entry and query head h
// (key/value head g = h / G), with chunks of B tokens and nch chunks:
//     O[t]   = causal softmax attention of t over the tokens of its own chunk   (within-chunk term)
//            + Q[t]^T A_c(t)                                                    (retrieval term)
//     F_c    = K_c^T V_c                                  chunk state, d x d (tokens s < n)
//     W[c,:] = softmax over c' < c of scale * R_c . H_c'  meta attention over strictly earlier chunks
//     A_c    = sum over c' < c of W[c, c'] F_c'           retrieved state (chunk 0 retrieves nothing)
// R (meta queries, per query head) and H (meta keys, per key/value head) are inputs, one d-vector
// per chunk.
//
// How (gfx950; four kernels, every input read once, intermediates in fp32):
//  * bsbr_state_kernel: one work-group per (batch, kv head, chunk).  K and V of the chunk go to
//    LDS (rows past n zero-filled); F = K^T V on the matrix cores (bf16 products are exact in the
//    fp32 accumulator), both operands read transposed by the LDS unit (ds_read_b64_tr_b16).  F is
//    stored as 32 x 32 fp32 tiles in the accumulator's order: element (i, j) of tile
//    (i / 32, j / 32) sits at [(tile * 32 + j % 32) * 32 + i % 32], tile = (i / 32) * d / 32 + j / 32.
//  * bsbr_meta_kernel: one wavefront per (batch, query head, chunk): dot products of R_c with the
//    earlier H rows, max and sum across the wavefront, and the row of W stored transposed.
//  * bsbr_mix_kernel: A = W F as a small fp32 GEMM per (batch, query head) over the flattened
//    d*d states (layout-agnostic): a work-group takes 16 chunks x 64 state elements, its four
//    wavefronts split the earlier chunks and their partials are summed in LDS in a fixed order;
//    the group's weights are staged in LDS with one coalesced pass.
//  * bsbr_chunk_kernel: one work-group per (batch, query head, chunk), one wavefront per 32
//    queries: the within-chunk attention (exact softmax over the chunk's keys) and the retrieval
//    read-out on the matrix cores, with A_c split into two bf16 parts, and one output store.

#include "bwd_common.hpp"
#include "lane_ops.hpp"

namespace bsa {
namespace {

using namespace bwd;

template <int D, int BLK>
__global__ __launch_bounds__(256) void bsbr_state_kernel(BsbrParams p) {
    __shared__ __attribute__((aligned(1024))) __bf16 sK[BLK * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV[BLK * D];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t w = blockIdx.x;  // (b * heads_kv + g) * nch + c
    const int c = (int)(w % p.nch);
    const int64_t bg = w / p.nch;
    const int64_t n = p.n, t0 = (int64_t)c * BLK;
    const int rows = (int)((n - t0) < BLK ? (n - t0) : BLK);
    const __bf16* K = (const __bf16*)p.k + (bg * n + t0) * D;
    const __bf16* V = (const __bf16*)p.v + (bg * n + t0) * D;
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    for (int x = tid; x < BLK * CPR; x += 256) {
        const int r = x / CPR, cc = x % CPR;
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
        const uint4 kx = r < rows ? *(const uint4*)(K + (int64_t)r * D + cc * 8) : zero;
        const uint4 vx = r < rows ? *(const uint4*)(V + (int64_t)r * D + cc * 8) : zero;
        *(uint4*)(sK + Sw2<D>::off(r, cc)) = kx;
        *(uint4*)(sV + Sw2<D>::off(r, cc)) = vx;
    }
    __syncthreads();
    constexpr int NT = D / 32;            // 32-wide tiles per dimension
    constexpr int TPW = NT * NT / 4;      // tiles per wavefront
    const int hf = lane >> 5;
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    float* Fo = p.F + w * (int64_t)(D * D);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tile = wv * TPW + u, mb = tile / NT, nb = tile % NT;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < BLK / 16; ++ks) {
            // A: rows i of K^T (columns of K), B: columns j of V; both with 16 tokens as k, read in
            // the same (accumulator-layout) token order
            const bf16x8 a = t_fragment<D>(sK, 16 * ks + vr_lane, 32 * mb + vc_lane);
            const bf16x8 b = t_fragment<D>(sV, 16 * ks + vr_lane, 32 * nb + vc_lane);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        // lane holds column j = 32 nb + lane % 32 and rows i = 32 mb + 8 r4 + 4 hf + (0..3)
        float* T = Fo + ((int64_t)tile * 32 + (lane & 31)) * 32 + 4 * hf;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *(float4*)(T + 8 * r4) = make_float4(acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]);
    }
}

template <int D>
__global__ __launch_bounds__(64) void bsbr_meta_kernel(BsbrParams p) {
    const int lane = threadIdx.x;
    const int64_t w = blockIdx.x;  // (b * heads_q + h) * nch + c
    const int nch = p.nch;
    const int c = (int)(w % nch);
    const int64_t bh = w / nch, b = bh / p.heads_q, h = bh % p.heads_q;
    const int G = p.heads_q / p.heads_kv;
    const __bf16* Rc = (const __bf16*)p.r + w * D;
    const __bf16* Hg = (const __bf16*)p.h + (b * p.heads_kv + h / G) * (int64_t)nch * D;
    float rv[D];
#pragma unroll
    for (int x = 0; x < D / 8; ++x) {
        const uint4 u = *(const uint4*)(Rc + 8 * x);
        const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            rv[8 * x + 2 * y] = __uint_as_float(wds[y] << 16);
            rv[8 * x + 2 * y + 1] = __uint_as_float(wds[y] & 0xffff0000u);
        }
    }
    auto score = [&](int cp) {  // scale * R_c . H_cp, log2 units
        const __bf16* Hr = Hg + (int64_t)cp * D;
        float s = 0.f;
#pragma unroll
        for (int x = 0; x < D / 8; ++x) {
            const uint4 u = *(const uint4*)(Hr + 8 * x);
            const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                s = fmaf(rv[8 * x + 2 * y], __uint_as_float(wds[y] << 16), s);
                s = fmaf(rv[8 * x + 2 * y + 1], __uint_as_float(wds[y] & 0xffff0000u), s);
            }
        }
        return s * p.scale_log2;
    };
    float mx = -INFINITY;
    for (int cp = lane; cp < c; cp += 64) mx = fmaxf(mx, score(cp));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.f;
    for (int cp = lane; cp < c; cp += 64) sum += __builtin_amdgcn_exp2f(score(cp) - mx);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    const float inv = c > 0 ? 1.f / sum : 0.f;
    // stored transposed, W^T[c'][c], so that the mix reads the weights of consecutive chunks c
    // for one earlier chunk c' as one scalar load
    float* Wt = p.W + bh * nch * (int64_t)nch + c;
    for (int cp = lane; cp < nch; cp += 64)
        Wt[(int64_t)cp * nch] = cp < c ? __builtin_amdgcn_exp2f(score(cp) - mx) * inv : 0.f;
}

constexpr int kMixRows = 16;   // chunks per work-group (accumulators per thread)
constexpr int kMixCols = 64;   // state elements per work-group (one per lane)
constexpr int kMixPf = 8;      // earlier chunks per wavefront step (their loads issued together)

// A[c][e] = sum over c' < c of W[c][c'] F[c'][e].  Work-group = 16 chunks c x 64 state elements e;
// its 4 wavefronts split the earlier chunks c' (wavefront w takes c' = w mod 4) so that each
// lane's chain of dependent loads is a quarter as long, and sum their partials in LDS in a fixed
// order.  The group's weights (16 per earlier chunk, contiguous in W^T) are staged in LDS once
// and read back as broadcasts.
__global__ __launch_bounds__(256) void bsbr_mix_kernel(BsbrParams p, int dd) {
    __shared__ float part[4][kMixRows][kMixCols];
    extern __shared__ __attribute__((aligned(16))) float sWt[];  // [c' < cmax][16]
    const int nch = p.nch;
    const int slices = dd / kMixCols;
    const int groups = (nch + kMixRows - 1) / kMixRows;
    const int64_t w = blockIdx.x;
    const int slice = (int)(w % slices);
    const int grp = (int)((w / slices) % groups);
    const int64_t bh = w / slices / groups;
    const int64_t b = bh / p.heads_q, h = bh % p.heads_q;
    const int G = p.heads_q / p.heads_kv;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = grp * kMixRows;
    const int rows = (nch - c0) < kMixRows ? nch - c0 : kMixRows;
    const int cmax = c0 + rows - 1;  // the group's last chunk reads chunks c' < cmax
    const int e = slice * kMixCols + lane;
    const float* Fg = p.F + (b * p.heads_kv + h / G) * (int64_t)nch * dd + e;
    // W^T row c' for this group: Wt[c' * nch + c0 .. + 16].  All 16 are read even when the group
    // has fewer chunks (the workspace pads W by 16 floats); the extra rows are never stored.
    const float* Wt = p.W + bh * nch * (int64_t)nch + c0;
    for (int x = threadIdx.x; x < cmax * kMixRows; x += 256)
        sWt[x] = Wt[(int64_t)(x / kMixRows) * nch + x % kMixRows];
    __syncthreads();
    float acc[kMixRows];
#pragma unroll
    for (int u = 0; u < kMixRows; ++u) acc[u] = 0.f;
    for (int cb = wv; cb < cmax; cb += 4 * kMixPf) {
        float f[kMixPf];
#pragma unroll
        for (int y = 0; y < kMixPf; ++y) {
            const int cp = cb + 4 * y;
            f[y] = cp < cmax ? Fg[(int64_t)cp * dd] : 0.f;
        }
#pragma unroll
        for (int y = 0; y < kMixPf; ++y) {
            const int cp = cb + 4 * y;
            if (cp >= cmax) break;
            const float4* wr = (const float4*)(sWt + cp * kMixRows);
#pragma unroll
            for (int q4 = 0; q4 < kMixRows / 4; ++q4) {
                const float4 wq = wr[q4];
                acc[4 * q4] = fmaf(wq.x, f[y], acc[4 * q4]);
                acc[4 * q4 + 1] = fmaf(wq.y, f[y], acc[4 * q4 + 1]);
                acc[4 * q4 + 2] = fmaf(wq.z, f[y], acc[4 * q4 + 2]);
                acc[4 * q4 + 3] = fmaf(wq.w, f[y], acc[4 * q4 + 3]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kMixRows; ++u) part[wv][u][lane] = acc[u];
    __syncthreads();
    // wavefront w sums rows u = 4 w .. 4 w + 3 over the four partials, in order
    float* Ao = p.A + (bh * nch + c0) * (int64_t)dd + e;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
        const int u = 4 * wv + y;
        if (u < rows) Ao[(int64_t)u * dd] = ((part[0][u][lane] + part[1][u][lane]) + part[2][u][lane]) + part[3][u][lane];
    }
}

// The whole output of one chunk c for one query head: within-chunk causal attention plus the
// retrieval.  One wavefront per 32 queries (lane = query), K_c, V_c and A_c staged in LDS:
//   S^T = K_c Q^T (key blocks up to the wavefront's own; later ones are fully in the future),
//   exact softmax per query (the whole row is in the lane pair: in-lane max and sum plus one
//   exchange between the half-wavefronts), P rounded to bf16, O^T = V^T P^T / l with V^T read
//   transposed; then O^T += A_c^T Q^T on the matrix cores with A_c split into bf16 hi and lo
//   parts (the same Q fragments are the B operand), and one bf16 store.
template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) void bsbr_chunk_kernel(BsbrParams p) {
    constexpr int NW = BLK / 32;
    constexpr int NT = D / 32;
    __shared__ __attribute__((aligned(1024))) __bf16 sK[BLK * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV[BLK * D];
    __shared__ __attribute__((aligned(16))) float sA[D * D];  // A_c in the tile layout
    const int nch = p.nch;
    const int64_t w = blockIdx.x;  // (b * heads_q + h) * nch + c
    const int c = (int)(w % nch);
    const int64_t bh = w / nch, b = bh / p.heads_q, h = bh % p.heads_q;
    const int G = p.heads_q / p.heads_kv;
    const int64_t n = p.n, t0 = (int64_t)c * BLK;
    const int rows = (int)((n - t0) < BLK ? (n - t0) : BLK);
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    {
        const int64_t kv_row0 = (b * p.heads_kv + h / G) * n + t0;
        const __bf16* K = (const __bf16*)p.k + kv_row0 * D;
        const __bf16* V = (const __bf16*)p.v + kv_row0 * D;
        constexpr int CPR = D / 8;
        for (int x = tid; x < BLK * CPR; x += NW * 64) {
            const int r = x / CPR, cc = x % CPR;
            const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
            *(uint4*)(sK + Sw2<D>::off(r, cc)) = r < rows ? *(const uint4*)(K + (int64_t)r * D + cc * 8) : zero;
            *(uint4*)(sV + Sw2<D>::off(r, cc)) = r < rows ? *(const uint4*)(V + (int64_t)r * D + cc * 8) : zero;
        }
        if (c > 0) {
            const float* Ac = p.A + w * (int64_t)(D * D);
            for (int x = tid; x < D * D / 4; x += NW * 64) *(float4*)(sA + 4 * x) = *(const float4*)(Ac + 4 * x);
        }
    }
    const int qloc = 32 * wv + l32;  // this lane's query within the chunk
    const bool q_ok = qloc < rows;
    const __bf16* Qr = (const __bf16*)p.q + (bh * n + t0 + (q_ok ? qloc : 0)) * D;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = q_ok ? *(const bf16x8*)(Qr + 16 * kk + 8 * hf) : bf16x8{};
    __syncthreads();

    // scores S^T[key][query] of the key blocks kb <= wv (rows 8 r4 + 4 hf + e of block kb)
    f32x16 s[NW];
#pragma unroll
    for (int kb = 0; kb < NW; ++kb) {
        s[kb] = f32x16{};
        if (kb <= wv) {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_fragment<D>(sK, 32 * kb + l32, 2 * kk + hf), qf[kk],
                                                                s[kb], 0, 0, 0);
        }
    }
    // causal mask (key <= query, key < n), max, exponentials in the log2 domain
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NW; ++kb) {
        if (kb > wv) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            const float v = (key <= qloc && key < rows) ? s[kb][r] * p.scale_log2 : -INFINITY;
            s[kb][r] = v;
            mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, lanes::xor_lane<32>(mx));
    float l = 0.f;
    uint32_t pk[NW][8];
#pragma unroll
    for (int kb = 0; kb < NW; ++kb) {
        if (kb > wv) continue;
#pragma unroll
        for (int r2 = 0; r2 < 8; ++r2) {
            pk[kb][r2] = pack_bf16x2(__builtin_amdgcn_exp2f(s[kb][2 * r2] - mx), __builtin_amdgcn_exp2f(s[kb][2 * r2 + 1] - mx));
            l = dot2_bf16_ones(pk[kb][r2], l);  // the sum of the weights as rounded for the product
        }
    }
    l += lanes::xor_lane<32>(l);
    // O^T[d][query] = V^T P^T: 16-key slices sl of block kb, keys in the accumulator order
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    f32x16 acc[NT];
#pragma unroll
    for (int db = 0; db < NT; ++db) acc[db] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < NW; ++kb) {
        if (kb > wv) continue;
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const bf16x8 bp = __builtin_bit_cast(
                bf16x8, make_uint4(pk[kb][4 * sl], pk[kb][4 * sl + 1], pk[kb][4 * sl + 2], pk[kb][4 * sl + 3]));
#pragma unroll
            for (int db = 0; db < NT; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    t_fragment<D>(sV, 32 * kb + 16 * sl + vr_lane, 32 * db + vc_lane), bp, acc[db], 0, 0, 0);
        }
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int db = 0; db < NT; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= inv;
    // retrieval: O^T[j][query] += sum_i A_c[i][j] Q[query][i]
    if (c > 0) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const int i0 = 16 * ks + 8 * hf;  // this lane's 8 values of i
#pragma unroll
            for (int nb = 0; nb < NT; ++nb) {
                // A_c^T row j = 32 nb + l32, i = i0 .. i0 + 7: tile (i / 32, j / 32), offset j % 32, i % 32
                const float* src = sA + ((i0 / 32) * NT + nb) * 1024 + l32 * 32 + (i0 % 32);
                const float4 a0 = *(const float4*)src, a1 = *(const float4*)(src + 4);
                const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                bf16x8 ahi, alo;
#pragma unroll
                for (int y = 0; y < 8; ++y) {
                    ahi[y] = (__bf16)av[y];
                    alo[y] = (__bf16)(av[y] - (float)ahi[y]);
                }
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, qf[ks], acc[nb], 0, 0, 0);
                acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, qf[ks], acc[nb], 0, 0, 0);
            }
        }
    }
    if (!q_ok) return;
    // lane holds its query and columns j = 32 db + 8 r4 + 4 hf + (0..3)
    __bf16* Or = (__bf16*)p.o + (bh * n + t0 + qloc) * D;
#pragma unroll
    for (int db = 0; db < NT; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *(uint2*)(Or + 32 * db + 8 * r4 + 4 * hf) =
                make_uint2(pack_bf16x2(acc[db][4 * r4], acc[db][4 * r4 + 1]), pack_bf16x2(acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]));
}

template <int D, int BLK>
hipError_t launch_t(const BsbrParams& p, hipStream_t stream) {
    const int64_t q_chunks = (int64_t)p.batch * p.heads_q * p.nch;
    hipLaunchKernelGGL((bsbr_state_kernel<D, BLK>), dim3((unsigned)((int64_t)p.batch * p.heads_kv * p.nch)), dim3(256), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bsbr_meta_kernel<D>), dim3((unsigned)q_chunks), dim3(64), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.nch > 1) {
        const int dd = D * D, slices = dd / kMixCols, groups = (p.nch + kMixRows - 1) / kMixRows;
        // dynamic LDS: the staged weights, at most 16 x (nch - 1) floats (<= 64 KiB at 1024 chunks)
        const size_t lds = (size_t)kMixRows * (p.nch - 1) * sizeof(float);
        hipLaunchKernelGGL(bsbr_mix_kernel, dim3((unsigned)((int64_t)p.batch * p.heads_q * groups * slices)),
                           dim3(256), lds, stream, p, dd);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bsbr_chunk_kernel<D, BLK>), dim3((unsigned)q_chunks), dim3(BLK / 32 * 64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bsbr(const BsbrParams& p, int d, int chunk, hipStream_t stream) {
    if (d == 128) return chunk == 128 ? launch_t<128, 128>(p, stream) : launch_t<128, 64>(p, stream);
    return chunk == 128 ? launch_t<64, 128>(p, stream) : launch_t<64, 64>(p, stream);
}

}  // namespace bsa
