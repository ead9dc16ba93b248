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
// How (gfx950; three kernels, every input read once, intermediates in fp32):
//  * bsbr_state_kernel: one work-group per (batch, kv head, chunk).  K and V of the chunk go to
//    LDS (rows past n zero-filled); F = K^T V on the matrix cores (bf16 products are exact in the
//    fp32 accumulator), both operands read transposed by the LDS unit (ds_read_b64_tr_b16).  F is
//    stored as 32 x 32 fp32 tiles in the accumulator's order: element (i, j) of tile
//    (i / 32, j / 32) sits at [(tile * 32 + j % 32) * 32 + i % 32], tile = (i / 32) * d / 32 + j / 32.
//  * bsbr_mix_kernel: per (batch, query head, 32 chunks, 128 of the flattened d*d state
//    elements): the meta scores of the 32 chunks against the earlier ones on the matrix cores,
//    their softmax in LDS, then A = W F with the fp32 matrix-core product (F rows read once per
//    32-chunk tile, coalesced).
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

constexpr int kMixE = 128;  // flattened state elements per work-group: 4 wavefronts x 32
constexpr int kMixKB = 64;  // earlier chunks per block of the A = W F product

// Position of earlier chunk c' in an LDS row of weights: within each block of 64, the even
// chunks first, then the odd ones, so that a lane's operands of one block (chunks k0 + 2 y + hf,
// y = 0..31) are 32 consecutive floats.
__device__ inline int mix_pos(int cp) { return (cp & ~63) + ((cp & 1) << 5) + ((cp & 63) >> 1); }

// The retrieved states of 32 consecutive chunks c0 .. c0 + 31 for one (batch, query head), over
// 128 of the d*d state elements (the sum is layout-agnostic over them):
//  1. meta scores S[i][c'] = scale R_{c0+i} . H_c' for every c' the tile's rows can see, on the
//     matrix cores (bf16 products are exact in the fp32 accumulator); wavefront w takes the
//     32-chunk column blocks w, w + 4, ...; the scores go to LDS rows (stride 4 mod 64 floats, so
//     that the 16-byte operand reads of step 3 are conflict-free);
//  2. the softmax numerators exp2(S - max) over c' < c0 + i in place (zero elsewhere) and the
//     row's 1 / sum (8 threads per row, 8 weights per LDS batch; row 0 of chunk 0 has no earlier
//     chunk and stays all zero);
//  3. A[c0 + i][e] = (1 / sum_i) sum over c' of exp[i][c'] F[c'][e] with the fp32 matrix-core
//     product v_mfma_f32_32x32x2_f32 (A operand: the numerators from LDS, B operand: F rows read
//     straight from global memory, 32 consecutive elements per half-wavefront, in blocks of 64
//     earlier chunks; the first block is requested at entry, so that its latency overlaps steps 1
//     and 2); two accumulators; wavefront w owns elements 32 w .. 32 w + 31 of the slice.
// Each work-group recomputes its 32 rows of meta scores (a few matrix-core instructions), so no
// weight matrix is stored.
template <int D>
__global__ __launch_bounds__(256) void bsbr_mix_kernel(BsbrParams p) {
    extern __shared__ __attribute__((aligned(16))) float sW[];  // [32][ldw], then 1 / sum [32]
    constexpr int DD = D * D;
    constexpr int slices = DD / kMixE;
    const int nch = p.nch;
    const int ldw = ((nch + 63) & ~63) + 4;
    float* sInv = sW + 32 * ldw;
    const int tiles = (nch + 31) / 32;
    const int64_t w = blockIdx.x;
    const int slice = (int)(w % slices);
    const int ct = (int)((w / slices) % tiles);
    const int64_t bh = w / slices / tiles;
    const int64_t b = bh / p.heads_q, h = bh % p.heads_q;
    const int64_t bg = b * p.heads_kv + h / (p.heads_q / p.heads_kv);
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c0 = 32 * ct;
    const int rows = (nch - c0) < 32 ? nch - c0 : 32;
    const int ncp = c0 + rows - 1;  // the tile's rows see the chunks c' < ncp
    const int ncp64 = (ncp + 63) & ~63;

    // F values of one block: chunk k0 + 2 y + hf, element e (zero past ncp)
    const int e = slice * kMixE + 32 * wv + l32;
    const float* Fg = p.F + bg * nch * (int64_t)DD + e;
    float f[kMixKB / 2];
    auto load_block = [&](int k0) {
#pragma unroll
        for (int y = 0; y < kMixKB / 2; ++y) {
            const int cp = k0 + 2 * y + hf;
            f[y] = cp < ncp ? Fg[(int64_t)cp * DD] : 0.f;
        }
    };
    load_block(0);

    // 1. meta scores of the tile's rows against chunks c' < ncp64 (zero past ncp)
    {
        const int rc = c0 + l32;
        const __bf16* Rr = (const __bf16*)p.r + (bh * nch + (l32 < rows ? rc : c0)) * D;
        bf16x8 rf[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) rf[kk] = l32 < rows ? *(const bf16x8*)(Rr + 16 * kk + 8 * hf) : bf16x8{};
        const __bf16* Hg = (const __bf16*)p.h + bg * nch * (int64_t)D;
        for (int cb = wv; 32 * cb < ncp64; cb += 4) {
            const int cp = 32 * cb + l32;  // this lane's column c'
            const __bf16* Hr = Hg + (int64_t)(cp < ncp ? cp : 0) * D;
            f32x16 acc = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const bf16x8 hv = cp < ncp ? *(const bf16x8*)(Hr + 16 * kk + 8 * hf) : bf16x8{};
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf[kk], hv, acc, 0, 0, 0);
            }
            // lane holds column cp at rows 8 (r / 4) + 4 hf + r % 4
            const int pc = mix_pos(cp);
#pragma unroll
            for (int r = 0; r < 16; ++r) sW[(8 * (r >> 2) + 4 * hf + (r & 3)) * ldw + pc] = acc[r] * p.scale_log2;
        }
    }
    __syncthreads();
    // 2. numerators exp2(S - max) for c' < c0 + i, zero for the other positions < ncp64; 1 / sum.
    //    Thread (i, part) takes positions 8 part + 64 m + (0..7), m = 0, 1, ... (two float4s).
    {
        const int i = tid >> 3, part = tid & 7;
        const int len = i < rows ? c0 + i : 0;
        float* row = sW + i * ldw;
        auto chunk_of = [](int pos) { return (pos & ~63) + 2 * (pos & 31) + ((pos >> 5) & 1); };
        float mx = -INFINITY;
        for (int p0 = 8 * part; p0 < ncp64; p0 += 64) {
            const float4 a = *(const float4*)(row + p0), z = *(const float4*)(row + p0 + 4);
            const float v[8] = {a.x, a.y, a.z, a.w, z.x, z.y, z.z, z.w};
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (chunk_of(p0 + u) < len) mx = fmaxf(mx, v[u]);
        }
        // max and sum over the row's 8 consecutive lanes by DPP (no LDS round trips)
        mx = fmaxf(mx, lanes::xor_lane<1>(mx));
        mx = fmaxf(mx, lanes::xor_lane<2>(mx));
        mx = fmaxf(mx, lanes::half_mirror(mx));
        float sum = 0.f;
        for (int p0 = 8 * part; p0 < ncp64; p0 += 64) {
            const float4 a = *(const float4*)(row + p0), z = *(const float4*)(row + p0 + 4);
            const float v[8] = {a.x, a.y, a.z, a.w, z.x, z.y, z.z, z.w};
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                x[u] = chunk_of(p0 + u) < len ? __builtin_amdgcn_exp2f(v[u] - mx) : 0.f;
                sum += x[u];
            }
            *(float4*)(row + p0) = make_float4(x[0], x[1], x[2], x[3]);
            *(float4*)(row + p0 + 4) = make_float4(x[4], x[5], x[6], x[7]);
        }
        sum = lanes::group_sum<8>(sum);
        if (part == 0) sInv[i] = len > 0 ? 1.f / sum : 0.f;
    }
    __syncthreads();
    // 3. A = (1 / sum) exp F over c' < ncp, two earlier chunks per instruction (k = hf)
    f32x16 acc0 = f32x16{}, acc1 = f32x16{};
    const float* Wr = sW + l32 * ldw + 32 * hf;
    for (int k0 = 0;;) {
        float wa[kMixKB / 2];
#pragma unroll
        for (int y4 = 0; y4 < kMixKB / 8; ++y4) {
            const float4 t = *(const float4*)(Wr + k0 + 4 * y4);
            wa[4 * y4] = t.x;
            wa[4 * y4 + 1] = t.y;
            wa[4 * y4 + 2] = t.z;
            wa[4 * y4 + 3] = t.w;
        }
#pragma unroll
        for (int y = 0; y < kMixKB / 2; y += 2) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[y], f[y], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[y + 1], f[y + 1], acc1, 0, 0, 0);
        }
        k0 += kMixKB;
        if (k0 >= ncp) break;
        load_block(k0);
    }
    // lane holds element e at rows i = 8 (r / 4) + 4 hf + r % 4 of the tile
    float* Ao = p.A + (bh * nch + c0) * (int64_t)DD + e;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * hf + (r & 3);
        if (i < rows) Ao[(int64_t)i * DD] = (acc0[r] + acc1[r]) * sInv[i];
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
__global__ __launch_bounds__(BLK / 32 * 64) __attribute__((amdgpu_waves_per_eu(4))) void bsbr_chunk_kernel(BsbrParams p) {
    constexpr int NW = BLK / 32;
    constexpr int NT = D / 32;
    __shared__ __attribute__((aligned(1024))) __bf16 sK[BLK * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV[BLK * D];
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
        // A_c read straight from global memory (the four wavefronts share it through the caches),
        // so that LDS holds only K_c and V_c and four work-groups fit a CU
        const float* Ac = p.A + w * (int64_t)(D * D);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const int i0 = 16 * ks + 8 * hf;  // this lane's 8 values of i
#pragma unroll
            for (int nb = 0; nb < NT; ++nb) {
                // A_c^T row j = 32 nb + l32, i = i0 .. i0 + 7: tile (i / 32, j / 32), offset j % 32, i % 32
                const float* src = Ac + ((i0 / 32) * NT + nb) * 1024 + l32 * 32 + (i0 % 32);
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
    if (p.nch > 1) {
        // dynamic LDS: the meta scores / weights of 32 chunks, 32 rows of (nch rounded up to 64)
        // + 4 floats, and 32 row factors (about 129 KiB at 1024 chunks)
        const size_t lds = ((size_t)32 * (((p.nch + 63) & ~63) + 4) + 32) * sizeof(float);
        if (lds > 65536 &&
            (e = hipFuncSetAttribute((const void*)bsbr_mix_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds)) != hipSuccess)
            return e;
        const int64_t tiles = (p.nch + 31) / 32;
        hipLaunchKernelGGL((bsbr_mix_kernel<D>), dim3((unsigned)((int64_t)p.batch * p.heads_q * tiles * (D * D / kMixE))),
                           dim3(256), lds, stream, p);
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
