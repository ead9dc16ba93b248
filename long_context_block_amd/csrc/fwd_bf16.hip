// fwd_bf16.hip — bfloat16 block-sparse attention forward on gfx950 matrix cores.
//
// What it computes: for every (batch, query head, query block i), exact softmax attention of
// the block's queries over the keys of the key blocks listed in row i of the CSR route, with
// the causal mask inside the diagonal block ("Block-Sparse Attention", "Math Or Compute
// Schema": mask before softmax; "BF1 ...", Method: each query block reads itself causally).
// Skipped key blocks are never loaded or scored ("Block-Sparse Attention", "How It Works").
//
// How (gfx950 design, not the pages' Blackwell kernel):
//  * Work item = (batch, GP query heads that share one key/value head, query block i).  One
//    work-group of BLK/32 wavefronts; wavefront w owns query rows [32w, 32w+32) of the block
//    for all GP heads, so every K/V tile read from LDS feeds GP matrix products (GQA sharing).
//  * Loop over the row's key blocks ("Block Sparse Attention in LLMs", section 6).  K and V
//    tiles of BLK x D are copied HBM -> LDS one tile ahead with asynchronous direct-to-LDS
//    loads (global_load_lds_dwordx4, no register staging) into a double-buffered stage, one
//    barrier per tile.  Both stay row-major [key][d], XOR-swizzled in 16-byte chunks so that
//    the matrix-core operand reads are bank-conflict-free; V is read transposed by the LDS
//    unit itself (ds_read_b64_tr_b16).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (K from LDS
//    as the A operand, Q resident in registers as the B operand).  Each lane then holds one
//    query's scores, so the row max/sum are in-lane plus one exchange between the two
//    half-wavefronts; the exponentials, packed to bf16, are directly the B operand of
//    O^T += V^T P^T (V^T from LDS as the A operand).  No LDS round trip for P.
//  * Online softmax ("Block Sparse Attention in LLMs", section 7: tile, never materialise the
//    n x n matrix) in the log2 domain with exp2; the running max is only raised when a tile's
//    max exceeds it by more than kRescaleSlack (the final division by the running sum makes
//    the result independent of which max was used), so the O rescale is rare.
//  * Work-group order: longest rows first (every route kind here has row length growing with
//    i), and consecutive work items of one head slice are packed onto one XCD so that
//    concurrently resident work-groups of that XCD share K/V tiles in its L2.

#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kRescaleSlack = 8.0f;  // log2 units: P values stay <= 2^8 between rescales

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float dot2_bf16_ones(uint32_t packed, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

template <int D, int BLK, int GP>
struct Tile {
    static constexpr int NW = BLK / 32;               // wavefronts per work-group
    static constexpr int NT = NW * 64;                // threads per work-group
    static constexpr int KCH = D / 8;                 // 16-byte chunks per K/V row
    static constexpr int NI = BLK * D / 8 / 64;       // 1 KiB direct-to-LDS loads per tile and tensor
    static constexpr int NI_W = NI / NW;              // ... per wavefront
    static_assert(NI_W * NW == NI, "tile split");

    // K stage [key][d]: 16-byte chunk c of row r at chunk c ^ kswz(r) -> the S^T operand reads
    // (32 consecutive rows, one chunk) hit distinct banks.
    __device__ static inline int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    // V stage [key][d]: chunk c of row r at chunk c ^ vswz(r) -> the transposing reads (4
    // consecutive rows x 32 columns per half-wavefront) hit distinct banks.
    __device__ static inline int vswz(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
    __device__ static inline int k_off(int r, int c) { return r * D + ((c ^ kswz(r)) << 3); }
    __device__ static inline int v_off(int r, int col) { return r * D + ((((col >> 3) ^ vswz(r))) << 3) + (col & 7); }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D, int BLK, int GP>
__global__ __launch_bounds__(BLK / 32 * 64) void fwd_bf16_kernel(FwdParams p) {
    using T = Tile<D, BLK, GP>;
    // keys per online-softmax step: 64, or 32 when GP*D is large (keeps scores in registers)
    constexpr int NC = (GP * D >= 256) ? 1 : 2;
    constexpr int KS = 32 * NC;
    // Two stages as four distinct arrays: with the tile loop unrolled by two, every access names
    // its array at compile time, so the compiler can see that the asynchronous copy into one
    // stage never aliases the operand reads from the other (no stall on the prefetch).
    __shared__ __attribute__((aligned(1024))) __bf16 sK0[BLK * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV0[BLK * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sK1[BLK * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV1[BLK * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    // ---- work item ----------------------------------------------------------------------
    const int64_t nqb = p.nqb;
    const int hgroups = p.heads_q / GP;
    const int64_t total = (int64_t)p.batch * hgroups * nqb;
    const int64_t w = blockIdx.x;
    const int64_t vi = (total % 8 == 0) ? (w % 8) * (total / 8) + w / 8 : w;
    const int64_t slice = vi / nqb;
    const int64_t i = nqb - 1 - (vi % nqb);
    const int64_t b = slice / hgroups;
    const int h0 = (int)(slice % hgroups) * GP;
    const int64_t kvh = h0 / (p.heads_q / p.heads_kv);
    const int64_t n = p.n;

    const __bf16* Kg = (const __bf16*)p.k + (b * p.heads_kv + kvh) * n * D;
    const __bf16* Vg = (const __bf16*)p.v + (b * p.heads_kv + kvh) * n * D;

    const int qloc = 32 * wv + l32;  // query row within the block
    const int64_t qrow = i * BLK + qloc;
    const bool row_ok = qrow < n;

    // ---- Q fragments (B operand of S^T = K Q^T): Q[row][16kk + 8hf .. +8] ------------------
    bf16x8 qf[GP][D / 16];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const __bf16* Qg = (const __bf16*)p.q + ((b * p.heads_q + h0 + g) * n + qrow) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            if (row_ok) qf[g][kk] = *(const bf16x8*)(Qg + 16 * kk + 8 * hf);
            else qf[g][kk] = bf16x8{};
        }
    }

    f32x16 acc[GP][D / 32];
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[g][db] = f32x16{};
    float m_run[GP], l_run[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) { m_run[g] = -INFINITY; l_run[g] = 0.f; }

    int64_t e0 = p.row_ptr[i], e1 = p.row_ptr[i + 1];
    e0 = e0 < 0 ? 0 : (e0 > p.nnz ? p.nnz : e0);
    e1 = e1 < e0 ? e0 : (e1 > p.nnz ? p.nnz : e1);
    const int L = (int)(e1 - e0);

    // ---- asynchronous HBM -> LDS copy of one K/V tile (global_load_lds_dwordx4) ------------
    // Instruction q of a tensor writes LDS chunks [64q, 64q+64) of the tile, lane-contiguous;
    // each lane fetches the global chunk that the swizzle places there.  Rows past n are
    // clamped to row n-1: they only ever meet masked (future) scores.
    auto issue = [&](int64_t j, __bf16* Kd, __bf16* Vd) {
#pragma unroll
        for (int u = 0; u < T::NI_W; ++u) {
            const int qi = wv * T::NI_W + u;
            const int P = 64 * qi + lane;
            const int r = P / T::KCH, ph = P % T::KCH;
            int64_t s = j * BLK + r;
            s = s < n ? s : n - 1;
            const int ck = ph ^ T::kswz(r), cv = ph ^ T::vswz(r);
            __builtin_amdgcn_global_load_lds((const void*)(Kg + s * D + ck * 8),
                                             (lds_void*)(Kd + qi * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(Vg + s * D + cv * 8),
                                             (lds_void*)(Vd + qi * 512), 16, 0, 0);
        }
    };
    // route entry loads return into a register; the wavefront-uniform value is taken (and
    // checked) only when the entry is used, one tile later, so the load never stalls.
    auto col_load = [&](int t) -> int { return p.col_idx[e0 + t]; };
    auto col_use = [&](int raw) -> int64_t {
        const int64_t j = __builtin_amdgcn_readfirstlane(raw);
        return (j < 0 || j > i) ? -1 : j;  // malformed (non-causal) entries are skipped
    };

    int64_t jn = (L > 0) ? col_use(col_load(0)) : -1;
    if (jn >= 0) issue(jn, sK0, sV0);

    // per-lane V^T operand addressing for the transposing reads
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // one K/V tile: scores, mask, online softmax, PV
    auto compute = [&](int64_t j, const __bf16* Ks, const __bf16* Vs) {
        const bool diag = (j == i);

#pragma nounroll
        for (int ks = 0; ks < BLK / KS; ++ks) {
            f32x16 sacc[GP][NC];
#pragma unroll
            for (int g = 0; g < GP; ++g)
#pragma unroll
                for (int c2 = 0; c2 < NC; ++c2) sacc[g][c2] = f32x16{};
            // S^T[key][query] for KS keys: NC column blocks of 32 keys
#pragma unroll
            for (int c2 = 0; c2 < NC; ++c2) {
                const int c = NC * ks + c2;
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const bf16x8 a = *(const bf16x8*)(Ks + T::k_off(32 * c + l32, 2 * kk + hf));
#pragma unroll
                    for (int g = 0; g < GP; ++g)
                        sacc[g][c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[g][kk], sacc[g][c2], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (diag) {
#pragma unroll
                for (int c2 = 0; c2 < NC; ++c2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = 32 * (NC * ks + c2) + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (key > qloc) {
#pragma unroll
                            for (int g = 0; g < GP; ++g) sacc[g][c2][r] = -INFINITY;
                        }
                    }
            }
            // running max (log2 domain), raised lazily and per query row: a row's result never
            // depends on another row's scores, not even in rounding
            float mnew[GP];
            bool need[GP];
            bool any_need = false;
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                float mx = -INFINITY;
#pragma unroll
                for (int c2 = 0; c2 < NC; ++c2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[g][c2][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                mnew[g] = mx * p.scale_log2;
                need[g] = mnew[g] > m_run[g] + kRescaleSlack;
                any_need |= need[g];
            }
            if (__any(any_need)) {
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    const float alpha = need[g] ? __builtin_amdgcn_exp2f(m_run[g] - mnew[g]) : 1.0f;
                    m_run[g] = need[g] ? mnew[g] : m_run[g];
                    l_run[g] *= alpha;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) acc[g][db] *= alpha;
                }
            }
            // P = exp2(s * scale*log2e - m), packed to bf16; row sums of the rounded P
            uint32_t pk[GP][NC][8];
#pragma unroll
            for (int g = 0; g < GP; ++g)
#pragma unroll
                for (int c2 = 0; c2 < NC; ++c2)
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[g][c2][2 * x], p.scale_log2, -m_run[g]));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[g][c2][2 * x + 1], p.scale_log2, -m_run[g]));
                        pk[g][c2][x] = pack_bf16x2(p0, p1);
                        l_run[g] = dot2_bf16_ones(pk[g][c2][x], l_run[g]);
                    }
            __builtin_amdgcn_sched_barrier(0);
            // O^T[d][query] += V^T[d][key] P^T[key][query]; V^T read transposed from the
            // row-major V stage with ds_read_b64_tr_b16 (4 keys x 1 column per lane and read)
#pragma unroll
            for (int c2 = 0; c2 < NC; ++c2) {
                const int c = NC * ks + c2;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    bf16x8 bop[GP];
#pragma unroll
                    for (int g = 0; g < GP; ++g) {
                        uint4 u4 = make_uint4(pk[g][c2][4 * s], pk[g][c2][4 * s + 1], pk[g][c2][4 * s + 2],
                                              pk[g][c2][4 * s + 3]);
                        bop[g] = __builtin_bit_cast(bf16x8, u4);
                    }
                    const int vrow = 32 * c + 16 * s + vr_lane;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const int vcol = 32 * db + vc_lane;
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4*)(Vs + T::v_off(vrow, vcol)));
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4*)(Vs + T::v_off(vrow + 8, vcol)));
                        const bf16x8 a = __builtin_bit_cast(
                            bf16x8, make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                               __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y));
#pragma unroll
                        for (int g = 0; g < GP; ++g)
                            acc[g][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[g], acc[g][db], 0, 0, 0);
                    }
                }
            }
        }
    };

    // route entries are read two tiles ahead so their load latency hides behind a tile
    int jnn = (L > 1) ? col_load(1) : -1;
    for (int t = 0; t < L; t += 2) {
        int64_t j = jn;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // stage 0 holds tile t; everyone is done reading stage 1
        if (t + 1 < L) {
            jn = col_use(jnn);
            if (jn >= 0) issue(jn, sK1, sV1);
            jnn = (t + 2 < L) ? col_load(t + 2) : -1;
        }
        if (j >= 0) compute(j, sK0, sV0);
        if (t + 1 >= L) break;
        j = jn;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // stage 1 holds tile t+1; everyone is done reading stage 0
        if (t + 2 < L) {
            jn = col_use(jnn);
            if (jn >= 0) issue(jn, sK0, sV0);
            jnn = (t + 3 < L) ? col_load(t + 3) : -1;
        }
        if (j >= 0) compute(j, sK1, sV1);
    }

    // ---- epilogue: O = acc / l, rounded to bf16; optional LSE ----------------------------
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const float lt = l_run[g] + __shfl_xor(l_run[g], 32);
        const float inv = 1.0f / lt;
        if (row_ok) {
            __bf16* Og = (__bf16*)p.o + ((b * p.heads_q + h0 + g) * n + qrow) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const int d0 = 32 * db + 8 * j4 + 4 * hf;
                    const uint32_t w0 = pack_bf16x2(acc[g][db][4 * j4] * inv, acc[g][db][4 * j4 + 1] * inv);
                    const uint32_t w1 = pack_bf16x2(acc[g][db][4 * j4 + 2] * inv, acc[g][db][4 * j4 + 3] * inv);
                    *(uint2*)(Og + d0) = make_uint2(w0, w1);
                }
            if (p.lse && hf == 0)
                p.lse[(b * p.heads_q + h0 + g) * n + qrow] = (m_run[g] + __log2f(lt)) * 0.69314718055994530942f;
        }
    }
}

template <int D, int BLK, int GP>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.batch * (p.heads_q / GP) * p.nqb;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BLK, GP>), dim3((unsigned)grid), dim3(BLK / 32 * 64), 0, stream, p);
    return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_gp(const FwdParams& p, hipStream_t stream) {
    const int G = p.heads_q / p.heads_kv;
    if (G % 2 == 0) return launch<D, BLK, 2>(p, stream);
    return launch<D, BLK, 1>(p, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, int block, hipStream_t stream) {
    if (d == 64 && block == 64) return launch_gp<64, 64>(p, stream);
    if (d == 64 && block == 128) return launch_gp<64, 128>(p, stream);
    if (d == 128 && block == 64) return launch_gp<128, 64>(p, stream);
    if (d == 128 && block == 128) return launch_gp<128, 128>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace bsa
