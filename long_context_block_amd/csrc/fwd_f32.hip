// fwd_f32.hip — float32 block-sparse attention forward (VALU FMA, fp32 throughout).
//
// One work-group per (batch, query head, 16 rows of query block i).  The work-group walks row i of the
// CSR route ("Block Sparse Attention in LLMs", section 6: for each query block, for each
// allowed key block), stages keys/values through LDS in chunks of 32 keys and keeps an online
// softmax per query row ("Block Sparse Attention in LLMs", section 7: tile the computation and
// never materialise the n x n matrix).  The causal mask is applied on the diagonal block only;
// every other allowed block is fully visible to all rows of the query block.
//
// fp32 has no bf16 rounding anywhere: scores, exponentials, the running max/sum and the output
// accumulator are float32, and exp is evaluated as exp2 of the score pre-multiplied by
// scale*log2(e).

#include "bsa_internal.hpp"
#include "lane_ops.hpp"

namespace bsa {
namespace {

constexpr int kF32Threads = 256;
constexpr int kKeyChunk = 32;
constexpr int kRows = 16;  // query rows per work-group: 16 threads per row

template <int D, int BLK>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(FwdParams p) {
    constexpr int TPR = kF32Threads / kRows;  // threads per query row (one DPP row of lanes)
    constexpr int DPT = D / TPR;              // output dims per thread (contiguous, read as float4)
    constexpr int PARTS = BLK / kRows;        // work-groups per query block
    __shared__ __attribute__((aligned(16))) float Kc[kKeyChunk][D];
    __shared__ __attribute__((aligned(16))) float Vc[kKeyChunk][D];

    const int tid = threadIdx.x;
    const int64_t nqb = p.nqb;
    const int rpart = blockIdx.x % PARTS;
    const int64_t wi = blockIdx.x / PARTS;
    const int64_t bh = wi / nqb;               // batch * heads_q + h
    const int64_t i = nqb - 1 - (wi % nqb);    // longest rows first (routes grow with i)
    const int64_t b = bh / p.heads_q;
    const int64_t h = bh % p.heads_q;
    const int64_t kvh = h / (p.heads_q / p.heads_kv);
    const float* Q = (const float*)p.q + (b * p.heads_q + h) * p.n * D;
    const float* K = (const float*)p.k + (b * p.heads_kv + kvh) * p.n * D;
    const float* V = (const float*)p.v + (b * p.heads_kv + kvh) * p.n * D;
    float* O = (float*)p.o + (b * p.heads_q + h) * p.n * D;

    const int rloc = rpart * kRows + tid / TPR;  // query row within the block
    const int sub = tid % TPR;
    const int64_t t = i * BLK + rloc;
    const bool row_ok = t < p.n;

    float q[DPT], acc[DPT];
#pragma unroll
    for (int x = 0; x < DPT; ++x) {
        q[x] = row_ok ? Q[t * D + sub * DPT + x] : 0.f;
        acc[x] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;

    int64_t e0 = p.row_ptr[i], e1 = p.row_ptr[i + 1];
    e0 = e0 < 0 ? 0 : (e0 > p.nnz ? p.nnz : e0);
    e1 = e1 < e0 ? e0 : (e1 > p.nnz ? p.nnz : e1);

    for (int64_t e = e0; e < e1; ++e) {
        const int64_t j = p.col_idx[e];
        if (j < 0 || j > i) continue;  // malformed entry: not causal, skip
        const bool diag = (j == i);
        for (int kc = 0; kc < BLK; kc += kKeyChunk) {
            __syncthreads();  // previous chunk fully consumed
            for (int x = tid; x < kKeyChunk * D / 4; x += kF32Threads) {
                const int r = x / (D / 4), c = 4 * (x % (D / 4));
                const int64_t s = j * BLK + kc + r;
                const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                *(float4*)&Kc[r][c] = (s < p.n) ? *(const float4*)&K[s * D + c] : z;
                *(float4*)&Vc[r][c] = (s < p.n) ? *(const float4*)&V[s * D + c] : z;
            }
            __syncthreads();
            float sc[kKeyChunk];
            float cmax = -INFINITY;
            bool has_nan = false;  // fmaxf drops NaN: a NaN score is tracked apart and poisons the row
#pragma unroll
            for (int r = 0; r < kKeyChunk; ++r) {
                float part = 0.f;
#pragma unroll
                for (int x = 0; x < DPT; x += 4) {
                    const float4 kv = *(const float4*)&Kc[r][sub * DPT + x];
                    part = fmaf(q[x], kv.x, part);
                    part = fmaf(q[x + 1], kv.y, part);
                    part = fmaf(q[x + 2], kv.z, part);
                    part = fmaf(q[x + 3], kv.w, part);
                }
                part = lanes::group_sum<TPR>(part);
                float s2 = part * p.scale_log2;
                if (diag && (kc + r > rloc)) s2 = -INFINITY;  // causal mask inside the diagonal block
                sc[r] = s2;
                cmax = fmaxf(cmax, s2);
                has_nan |= (s2 != s2);
            }
            if (cmax == -INFINITY && !has_nan) continue;  // whole chunk masked for this row
            const float m_new = has_nan ? NAN : fmaxf(m_run, cmax);  // NaN: running sum and output go NaN
            const float alpha = exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int x = 0; x < DPT; ++x) acc[x] *= alpha;
            m_run = m_new;
#pragma unroll
            for (int r = 0; r < kKeyChunk; ++r) {
                const float pr = exp2f(sc[r] - m_run);
                l_run += pr;
#pragma unroll
                for (int x = 0; x < DPT; x += 4) {
                    const float4 vv = *(const float4*)&Vc[r][sub * DPT + x];
                    acc[x] = fmaf(pr, vv.x, acc[x]);
                    acc[x + 1] = fmaf(pr, vv.y, acc[x + 1]);
                    acc[x + 2] = fmaf(pr, vv.z, acc[x + 2]);
                    acc[x + 3] = fmaf(pr, vv.w, acc[x + 3]);
                }
            }
        }
    }
    if (row_ok) {
        const float inv = 1.f / l_run;
#pragma unroll
        for (int x = 0; x < DPT; ++x) O[t * D + sub * DPT + x] = acc[x] * inv;
        if (p.lse && sub == 0) p.lse[bh * p.n + t] = (m_run + log2f(l_run)) * 0.69314718055994530942f;
    }
}

template <int D, int BLK>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.batch * p.heads_q * p.nqb * (BLK / kRows);
    hipLaunchKernelGGL((fwd_f32_kernel<D, BLK>), dim3((unsigned)grid), dim3(kF32Threads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int d, int block, hipStream_t stream) {
    if (d == 64 && block == 64) return launch<64, 64>(p, stream);
    if (d == 64 && block == 128) return launch<64, 128>(p, stream);
    if (d == 128 && block == 64) return launch<128, 64>(p, stream);
    if (d == 128 && block == 128) return launch<128, 128>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace bsa
