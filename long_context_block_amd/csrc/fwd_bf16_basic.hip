// fwd_bf16_basic.hip — unpipelined bfloat16 block-sparse attention forward on gfx950 matrix
// cores, for the shapes the pipelined kernel (fwd_bf16.hip) does not take: rows that average at
// most about a block and a half without a GQA pair (the block-diagonal route), where one work
// item per work-group beats the persistent walk.
//
// What it computes: for every (batch, query head, query block i), exact softmax attention of
// the block's queries over the keys of the key blocks listed in row i of the CSR route, with
// the causal mask inside the diagonal block ("Block-Sparse Attention", "Math Or Compute
// Schema": mask before softmax; "BF1 ...", Method: each query block reads itself causally).
// Skipped key blocks are never loaded or scored ("Block-Sparse Attention", "How It Works").
//
// How: one work-group per work item (batch, GP query heads sharing a key/value head, query
// block i), GP * BLK/32 wavefronts of 32 query rows each; K/V chunks of CK keys are copied
// HBM -> LDS one chunk ahead (global_load_lds_dwordx4) into a two-stage ring with one barrier
// per chunk; each softmax step (64 keys, or 32 with 32-key chunks) computes S^T = K Q^T on the
// matrix cores, the online softmax in registers (one query per lane), and O^T += V^T P^T with
// V^T read by the LDS transposing read.
// The steps of a wavefront run in sequence; the two wavefronts of a SIMD overlap each other.

#include "fwd_common.hpp"

namespace bsa {
namespace {

using namespace fwd;

// Work item of a launch of `total` work-groups over head slices of nqb query blocks each:
// longest rows (largest i) first, and consecutive work items of one head slice packed onto
// one XCD (work-groups are dispatched round-robin over the 8 XCDs) so that they share K/V
// tiles in that XCD's L2.
__device__ inline void grid_item(int64_t w, int64_t total, int64_t nqb, int64_t& slice, int64_t& i) {
    const int64_t vi = (total % 8 == 0) ? (w % 8) * (total / 8) + w / 8 : w;
    slice = vi / nqb;
    i = nqb - 1 - (vi % nqb);
}

constexpr int kChunkGqa = 128;  // LDS chunk (keys) of GQA work-groups (one per CU)

template <int D, int BLK, int GP, int CK>
struct CfgBasic {
    static constexpr int NWQ = BLK / 32;              // wavefronts per query head
    static constexpr int NW = NWQ * GP;               // wavefronts per work-group
    static constexpr int NT = NW * 64;                // threads per work-group
    static constexpr int CPT = BLK / CK;              // LDS chunks per key block
    static constexpr int NC2 = CK >= 64 ? 2 : 1;      // 32-key score accumulators per softmax step
    static constexpr int KS = 32 * NC2;               // keys per softmax step
    static constexpr int SPC = CK / KS;               // softmax steps per chunk
    static constexpr int KCH = D / 8;                 // 16-byte chunks per K/V row
    static constexpr int NI = CK * D / 8 / 64;        // 1 KiB direct-to-LDS loads per chunk and tensor
    static constexpr int NI_W = NI / NW;              // ... per wavefront
    static constexpr int NST = 2;                     // ring stages
    static_assert(NI_W * NW == NI, "chunk split");
    static_assert(CPT * CK == BLK && SPC * KS == CK, "chunking");
};

template <int D, int BLK, int GP, int CK>
__global__ __launch_bounds__(BLK / 32 * GP * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_bf16_basic_kernel(FwdParams p) {
    using C = CfgBasic<D, BLK, GP, CK>;
    using Z = Swz<D>;
    __shared__ __attribute__((aligned(1024))) __bf16 sK[C::NST][CK * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV[C::NST][CK * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    // ---- work item ----------------------------------------------------------------------
    int64_t slice, i;
    const int hgroups = p.heads_q / GP;
    grid_item(blockIdx.x, (int64_t)p.batch * hgroups * p.nqb, p.nqb, slice, i);
    const int64_t b = slice / hgroups;
    const int h0 = (int)(slice % hgroups) * GP;
    const int64_t kvh = h0 / (p.heads_q / p.heads_kv);
    const int64_t n = p.n;
    const int g = wv / C::NWQ;                      // this wavefront's head within the group
    const int64_t head = b * p.heads_q + h0 + g;    // flattened (batch, query head)

    const __bf16* Kg = (const __bf16*)p.k + (b * p.heads_kv + kvh) * n * D;
    const __bf16* Vg = (const __bf16*)p.v + (b * p.heads_kv + kvh) * n * D;

    const int qloc = 32 * (wv % C::NWQ) + l32;  // query row within the block
    const int64_t qrow = i * BLK + qloc;
    const bool row_ok = qrow < n;

    // ---- Q fragments (B operand of S^T = K Q^T): Q[row][16kk + 8hf .. +8] ------------------
    bf16x8 qf[D / 16];
    {
        const __bf16* Qr = (const __bf16*)p.q + (head * n + qrow) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) qf[kk] = row_ok ? *(const bf16x8*)(Qr + 16 * kk + 8 * hf) : bf16x8{};
    }

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    int64_t e0 = p.row_ptr[i], e1 = p.row_ptr[i + 1];
    e0 = e0 < 0 ? 0 : (e0 > p.nnz ? p.nnz : e0);
    e1 = e1 < e0 ? e0 : (e1 > p.nnz ? p.nnz : e1);
    const int L = (int)(e1 - e0);     // key blocks
    const int NCH = L * C::CPT;       // LDS chunks

    // Route entry loads return into a register; the wavefront-uniform value is taken (and
    // checked) only when the entry is used, a key block later, so the load never stalls.
    // (scalar loads through the constant address space: they are counted by lgkmcnt, not by the
    // vmcnt that tracks the asynchronous K/V copies)
    const __attribute__((address_space(4))) int32_t* cidx = (const __attribute__((address_space(4))) int32_t*)p.col_idx;
    auto col_load = [&](int t) -> int { return cidx[e0 + t]; };
    auto col_use = [&](int raw) -> int64_t {
        const int64_t j = __builtin_amdgcn_readfirstlane(raw);
        return (j < 0 || j > i) ? -1 : j;  // malformed (non-causal) entry: a fully masked chunk
    };
    // first global row of chunk `ch` of key block j (a skipped entry reads block i, all masked)
    auto chunk_row = [&](int64_t j, int ch) -> int64_t { return (j >= 0 ? j : i) * BLK + CK * (ch % C::CPT); };

    // ---- asynchronous HBM -> LDS copy of one chunk of CK keys -------------------------------
    // Instruction q of a tensor writes LDS chunks [64q, 64q+64) of the stage, lane-contiguous;
    // each lane fetches the global 16 bytes that the swizzle places there.  Rows past n are
    // clamped to row n-1: they only ever meet masked (future) scores.
    auto issue = [&](int64_t row0, int stage) {
#pragma unroll
        for (int u = 0; u < C::NI_W; ++u) {
            const int qi = wv * C::NI_W + u;
            const int P = 64 * qi + lane;
            const int r = P / C::KCH, ph = P % C::KCH;
            int64_t s = row0 + r;
            s = s < n ? s : n - 1;
            copy16_to_lds(Kg + s * D + (ph ^ Z::kswz(r)) * 8, lds_addr(&sK[stage][qi * 512]));
            copy16_to_lds(Vg + s * D + (ph ^ Z::vswz(r)) * 8, lds_addr(&sV[stage][qi * 512]));
        }
    };

    // per-lane V^T operand addressing for the transposing reads
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // ---- scores + online softmax of one chunk -> packed bf16 weights ---------------------
    // lim = largest visible key offset within the chunk for this lane's row (diagonal block)
    auto scores = [&](const __bf16* Ks, int krow0, bool masked, int lim, uint32_t (&pk)[2][8]) {
        f32x16 sacc[2];
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};  // (only the first NC2 are used)
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int c2 = 0; c2 < C::NC2; ++c2) {
                const bf16x8 a = *(const bf16x8*)(Ks + Z::k_off(krow0 + 32 * c2 + l32, 2 * kk + hf));
                sacc[c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[c2], 0, 0, 0);
            }
        if (masked) {  // only the diagonal block (or a skipped entry) masks anything (uniform)
#pragma unroll
            for (int c2 = 0; c2 < C::NC2; ++c2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * c2 + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (key > lim) sacc[c2][r] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int c2 = 0; c2 < C::NC2; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[c2][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = mx * p.scale_log2;
        const bool need = mnew > m_run + kRescaleSlack;
        if (__any(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
            m_run = need ? mnew : m_run;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
        }
        const float mo = (m_run == -INFINITY) ? 0.0f : m_run;  // fully masked so far: weights 0
        // P = exp2(s * scale*log2e - m), packed to bf16; row sums of the rounded P
#pragma unroll
        for (int c2 = 0; c2 < C::NC2; ++c2)
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[c2][2 * x], p.scale_log2, -mo));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[c2][2 * x + 1], p.scale_log2, -mo));
                pk[c2][x] = pack_bf16x2(p0, p1);
                l_run = dot2_bf16_ones(pk[c2][x], l_run);
            }
    };
    // ---- O^T[d][query] += V^T[d][key] P^T[key][query] over one softmax step -------------
    auto pv = [&](const __bf16* Vs, int vrow0, const uint32_t (&pk)[2][8]) {
#pragma unroll
        for (int c2 = 0; c2 < C::NC2; ++c2)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 bop = __builtin_bit_cast(
                    bf16x8, make_uint4(pk[c2][4 * s], pk[c2][4 * s + 1], pk[c2][4 * s + 2], pk[c2][4 * s + 3]));
                const int vrow = vrow0 + 32 * c2 + 16 * s + vr_lane;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 a = v_fragment<D>(Vs, vrow, 32 * db + vc_lane);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[db], 0, 0, 0);
                }
            }
    };

    // ---- chunk loop ------------------------------------------------------------------------
    if (L > 0) {
        int64_t jt = col_use(col_load(0));                  // key block of chunk ch
        int64_t jt1 = (L > 1) ? col_use(col_load(1)) : -1;  // the next key block
        int raw = (L > 2) ? col_load(2) : -1;
        issue(chunk_row(jt, 0), 0);
        uint32_t pk[2][8];
        int st = 0;  // stage of chunk ch
        for (int ch = 0; ch < NCH; ++ch) {
            const int t = ch / C::CPT, part = ch % C::CPT;
            if (part == 0 && ch > 0) {
                jt = jt1;
                jt1 = col_use(raw);
                raw = (t + 2 < L) ? col_load(t + 2) : -1;
            }
            // chunk ch has landed in stage st (this wavefront's copies; the barrier covers the
            // others') and every wavefront is done with the other stage, refilled next.
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (ch + 1 < NCH) issue(chunk_row(((ch + 1) / C::CPT == t) ? jt : jt1, ch + 1), st ^ 1);
#pragma unroll
            for (int sp = 0; sp < C::SPC; ++sp) {
                const int kb = CK * part + C::KS * sp;  // first key of this step within the block
                const int lim = (jt < 0) ? -1 : (jt == i ? qloc - kb : C::KS);
                scores(sK[st], C::KS * sp, jt < 0 || jt == i, lim, pk);
                pv(sV[st], C::KS * sp, pk);
            }
            st ^= 1;
        }
    }

    // ---- epilogue: O = acc / l, rounded to bf16; optional LSE ----------------------------
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / lt;
    if (row_ok) {
        __bf16* Or = (__bf16*)p.o + (head * n + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int d0 = 32 * db + 8 * j4 + 4 * hf;
                const uint32_t w0 = pack_bf16x2(acc[db][4 * j4] * inv, acc[db][4 * j4 + 1] * inv);
                const uint32_t w1 = pack_bf16x2(acc[db][4 * j4 + 2] * inv, acc[db][4 * j4 + 3] * inv);
                *(uint2*)(Or + d0) = make_uint2(w0, w1);
            }
        if (p.lse && hf == 0) p.lse[head * n + qrow] = (m_run + __log2f(lt)) * kLn2;
    }
}

template <int D, int BLK, int GP, int CK>
hipError_t launch_basic(const FwdParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.batch * (p.heads_q / GP) * p.nqb;
    hipLaunchKernelGGL((fwd_bf16_basic_kernel<D, BLK, GP, CK>), dim3((unsigned)grid), dim3(CfgBasic<D, BLK, GP, CK>::NT), 0,
                       stream, p);
    return hipGetLastError();
}

// GQA pairs share K/V chunks in one work-group of 2 * BLK/32 wavefronts.
template <int D, int BLK>
hipError_t launch_basic_gp(const FwdParams& p, hipStream_t stream) {
    const int G = p.heads_q / p.heads_kv;
    if (G % 2 == 0) return launch_basic<D, BLK, 2, (BLK < kChunkGqa ? BLK : kChunkGqa)>(p, stream);
    // 64-token blocks without a GQA pair: 32-key chunks halve the LDS ring (32 KiB at d = 128),
    // so twice as many of these short, latency-bound work-groups are resident per CU
    if (BLK == 64) return launch_basic<D, BLK, 1, 32>(p, stream);
    return launch_basic<D, BLK, 1, 64>(p, stream);
}

}  // namespace

hipError_t launch_fwd_bf16_basic(const FwdParams& p, int d, int block, hipStream_t stream) {
    if (d == 64 && block == 64) return launch_basic_gp<64, 64>(p, stream);
    if (d == 64 && block == 128) return launch_basic_gp<64, 128>(p, stream);
    if (d == 128 && block == 64) return launch_basic_gp<128, 64>(p, stream);
    if (d == 128 && block == 128) return launch_basic_gp<128, 128>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace bsa
