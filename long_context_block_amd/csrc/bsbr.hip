// bsbr.hip — the BSBR between-chunk retrieval term on gfx950.
//
// What it computes ("bsbr", Solution: the retrieval half of the combined formula), per batch
// entry and query head h (key/value head g = h / G), with chunks of B tokens and nch chunks:
//     F_c    = K_c^T V_c                                  chunk state, d x d (tokens s < n)
//     W[c,:] = softmax over c' < c of scale * R_c . H_c'  meta attention over strictly earlier chunks
//     A_c    = sum over c' < c of W[c, c'] F_c'           retrieved state
//     O[t]  += Q[t]^T A_c(t)                               added to the within-chunk attention
// R (meta queries, per query head) and H (meta keys, per key/value head) are inputs, one d-vector
// per chunk.  Chunk 0 retrieves nothing.
//
// How (gfx950; each step is small next to the within-chunk attention, so the design keeps every
// tensor read once and the arithmetic in fp32 where it is not exact):
//  * bsbr_state_kernel: one work-group per (batch, kv head, chunk).  K and V of the chunk go to
//    LDS (rows past n zero-filled); F = K^T V on the matrix cores (bf16 products are exact in the
//    fp32 accumulator), both operands read transposed by the LDS unit (ds_read_b64_tr_b16).  F is
//    stored as 32 x 32 fp32 tiles in the accumulator's order: element (i, j) of tile
//    (i / 32, j / 32) sits at [(tile * 32 + j % 32) * 32 + i % 32], tile = (i / 32) * d / 32 + j / 32.
//  * bsbr_meta_kernel: one wavefront per (batch, query head, chunk): dot products of R_c with the
//    earlier H rows, max and sum across the wavefront, and the full row of W (zeros at c' >= c).
//  * bsbr_mix_kernel: A = W F as a small GEMM per (batch, query head) over the flattened d*d
//    states (layout-agnostic): a work-group takes 16 chunks x 1024 state elements; the 16 rows of
//    W are staged in LDS transposed, so each earlier chunk's state slice is read once per group.
//  * bsbr_apply_kernel: one work-group per (batch, query head, chunk >= 1): A_c is staged in LDS
//    row-major, each thread holds one token's query (fp32) and adds Q[t]^T A_c to a slice of the
//    output row, which it reads, adds to and rounds to bf16 once more.

#include "bwd_common.hpp"

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
    float* Wr = p.W + w * nch;
    for (int cp = lane; cp < nch; cp += 64) Wr[cp] = cp < c ? __builtin_amdgcn_exp2f(score(cp) - mx) * inv : 0.f;
}

constexpr int kMixRows = 16;     // chunks per mix work-group
constexpr int kMixCols = 1024;   // state elements per mix work-group (4 per thread)

__global__ __launch_bounds__(256) void bsbr_mix_kernel(BsbrParams p, int dd) {
    extern __shared__ __attribute__((aligned(16))) float sW[];  // [c'][16]: W of the group's 16 chunks, transposed
    const int nch = p.nch;
    const int slices = dd / kMixCols;
    const int groups = (nch + kMixRows - 1) / kMixRows;
    const int64_t w = blockIdx.x;
    const int slice = (int)(w % slices);
    const int grp = (int)((w / slices) % groups);
    const int64_t bh = w / slices / groups;
    const int64_t b = bh / p.heads_q, h = bh % p.heads_q;
    const int G = p.heads_q / p.heads_kv;
    const int c0 = grp * kMixRows;
    const int rows = (nch - c0) < kMixRows ? nch - c0 : kMixRows;
    const int cmax = c0 + rows - 1;  // earlier chunks of the group's last chunk: c' < cmax
    for (int x = threadIdx.x; x < kMixRows * cmax; x += 256) {
        const int u = x / cmax, cp = x % cmax;
        sW[cp * kMixRows + u] = u < rows ? p.W[(bh * nch + c0 + u) * nch + cp] : 0.f;
    }
    __syncthreads();
    const int e = slice * kMixCols + 4 * threadIdx.x;
    const float* Fg = p.F + (b * p.heads_kv + h / G) * (int64_t)nch * dd + e;
    float4 acc[kMixRows];
#pragma unroll
    for (int u = 0; u < kMixRows; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int cp = 0; cp < cmax; ++cp) {
        const float4 f = *(const float4*)(Fg + (int64_t)cp * dd);
        const float4* wr = (const float4*)(sW + cp * kMixRows);
#pragma unroll
        for (int q4 = 0; q4 < kMixRows / 4; ++q4) {
            const float4 wq = wr[q4];
            const float ws[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                float4& a = acc[4 * q4 + y];
                a.x = fmaf(ws[y], f.x, a.x);
                a.y = fmaf(ws[y], f.y, a.y);
                a.z = fmaf(ws[y], f.z, a.z);
                a.w = fmaf(ws[y], f.w, a.w);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kMixRows; ++u)
        if (u < rows) *(float4*)(p.A + (bh * nch + c0 + u) * (int64_t)dd + e) = acc[u];
}

template <int D, int BLK>
__global__ __launch_bounds__(256) void bsbr_apply_kernel(BsbrParams p) {
    __shared__ __attribute__((aligned(16))) float sA[D * D];  // A_c row-major [i][j]
    const int nch = p.nch;
    const int64_t w = blockIdx.x;  // (b * heads_q + h) * nch + c
    const int c = (int)(w % nch);
    if (c == 0) return;            // chunk 0 retrieves nothing
    const int64_t bh = w / nch;
    const int tid = threadIdx.x;
    constexpr int NT = D / 32;
    const float* Ac = p.A + w * (int64_t)(D * D);
    for (int x = tid; x < D * D / 4; x += 256) {  // tile layout -> row-major
        const float4 v = *(const float4*)(Ac + 4 * x);
        const int e = 4 * x, m = e % 32, nn = (e / 32) % 32, tile = e / 1024;
        const int i = 32 * (tile / NT) + m, j = 32 * (tile % NT) + nn;
        sA[(i + 0) * D + j] = v.x;
        sA[(i + 1) * D + j] = v.y;
        sA[(i + 2) * D + j] = v.z;
        sA[(i + 3) * D + j] = v.w;
    }
    __syncthreads();
    constexpr int TPT = 256 / BLK;  // threads per token
    constexpr int JS = D / TPT;     // output columns per thread
    const int64_t t = (int64_t)c * BLK + tid / TPT;
    if (t >= p.n) return;
    const int j0 = (tid % TPT) * JS;
    const __bf16* Qr = (const __bf16*)p.q + (bh * p.n + t) * D;
    float qv[D];
#pragma unroll
    for (int x = 0; x < D / 8; ++x) {
        const uint4 u = *(const uint4*)(Qr + 8 * x);
        const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            qv[8 * x + 2 * y] = __uint_as_float(wds[y] << 16);
            qv[8 * x + 2 * y + 1] = __uint_as_float(wds[y] & 0xffff0000u);
        }
    }
    float acc[JS];
#pragma unroll
    for (int j = 0; j < JS; ++j) acc[j] = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
        const float* ar = sA + i * D + j0;
#pragma unroll
        for (int j = 0; j < JS; j += 4) {
            const float4 a = *(const float4*)(ar + j);
            acc[j] = fmaf(qv[i], a.x, acc[j]);
            acc[j + 1] = fmaf(qv[i], a.y, acc[j + 1]);
            acc[j + 2] = fmaf(qv[i], a.z, acc[j + 2]);
            acc[j + 3] = fmaf(qv[i], a.w, acc[j + 3]);
        }
    }
    __bf16* Or = (__bf16*)p.o + (bh * p.n + t) * D + j0;
#pragma unroll
    for (int j = 0; j < JS; j += 8) {
        const uint4 u = *(const uint4*)(Or + j);
        const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
        uint32_t outw[4];
#pragma unroll
        for (int y = 0; y < 4; ++y)
            outw[y] = pack_bf16x2(__uint_as_float(wds[y] << 16) + acc[j + 2 * y],
                                  __uint_as_float(wds[y] & 0xffff0000u) + acc[j + 2 * y + 1]);
        *(uint4*)(Or + j) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
}

template <int D, int BLK>
hipError_t launch_t(const BsbrParams& p, hipStream_t stream) {
    const int64_t kv_chunks = (int64_t)p.batch * p.heads_kv * p.nch;
    const int64_t q_chunks = (int64_t)p.batch * p.heads_q * p.nch;
    hipLaunchKernelGGL((bsbr_state_kernel<D, BLK>), dim3((unsigned)kv_chunks), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bsbr_meta_kernel<D>), dim3((unsigned)q_chunks), dim3(64), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.nch > 1) {
        const int dd = D * D, slices = dd / kMixCols, groups = (p.nch + kMixRows - 1) / kMixRows;
        const size_t lds = (size_t)kMixRows * p.nch * sizeof(float);
        hipLaunchKernelGGL(bsbr_mix_kernel, dim3((unsigned)((int64_t)p.batch * p.heads_q * groups * slices)),
                           dim3(256), lds, stream, p, dd);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((bsbr_apply_kernel<D, BLK>), dim3((unsigned)q_chunks), dim3(256), 0, stream, p);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_bsbr_retrieval(const BsbrParams& p, int d, int chunk, hipStream_t stream) {
    if (d == 128) return chunk == 128 ? launch_t<128, 128>(p, stream) : launch_t<128, 64>(p, stream);
    return chunk == 128 ? launch_t<64, 128>(p, stream) : launch_t<64, 64>(p, stream);
}

}  // namespace bsa
