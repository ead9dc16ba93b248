// fwd_bf16.hip — bfloat16 block-sparse attention forward on gfx950 matrix cores.
//
// What it computes: for every (batch, query head, query block i), exact softmax attention of
// the block's queries over the keys of the key blocks listed in row i of the CSR route, with
// the causal mask inside the diagonal block ("Block-Sparse Attention", "Math Or Compute
// Schema": mask before softmax; "BF1 ...", Method: each query block reads itself causally).
// Key blocks not in the row are never loaded or scored ("Block-Sparse Attention", "How It Works").
//
// How (gfx950 design, not the pages' Blackwell kernel).  This kernel takes 128- and 64-token
// blocks with GQA pairs, and multi-head attention over rows longer than about a block and a
// half; fwd_bf16_basic.hip takes the rest.
//  * Work item = (batch, GP query heads that share one key/value head, query block i).  The
//    work-group has GP * B / 32 wavefronts; wavefront w owns query head w / (B / 32) and 32 rows
//    of the block, so every K/V chunk staged in LDS feeds all GP heads (GQA sharing) while each
//    wavefront keeps one head's state (<= 256 VGPRs): two wavefronts per SIMD (one 8-wavefront
//    work-group per CU at B = 128, two 4-wavefront ones at B = 64).  The launch is persistent: as many work-groups as fit the device, each walking a
//    serpentine share of the items (longest rows first, the items of an XCD's share from the
//    same heads so that its work-groups share K/V tiles in that XCD's L2).
//  * Loop over the row's key blocks ("Block Sparse Attention in LLMs", section 6), one
//    LDS chunk per block (128 keys, two softmax steps; or 64 keys, one step).  Chunks are copied HBM -> LDS one chunk ahead with
//    asynchronous direct-to-LDS loads (global_load_lds_dwordx4, no register staging) into
//    rings of two K stages and three V stages (a chunk's V outlives its K by one softmax step,
//    see below), one barrier per chunk; the rings run on across work items, so the next item's
//    first chunk is in flight during the current item's last.  K and V stay row-major
//    [key][d], XOR-swizzled in 16-byte chunks so that the matrix-core operand reads are
//    bank-conflict-free; V is read transposed by the LDS unit itself (ds_read_b64_tr_b16).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (K from LDS
//    as the A operand, Q resident in registers as the B operand), 64 keys per online-softmax
//    step.  Each lane then holds one query's scores, so the row max/sum are in-lane plus one
//    exchange between the two half-wavefronts (v_permlane32_swap); the exponentials, packed to
//    bf16, are directly the B operand of O^T += V^T P^T (V^T from LDS as the A operand).
//  * Software pipeline over the steps of the unmasked key blocks: the exponentials of step t-1
//    are interleaved, instruction by instruction, with the score products of step t, and the
//    P V product of step t-1 with the row max of step t, so the vector ALU and the matrix
//    cores of a wavefront work at the same time (the other wavefront of the SIMD fills the
//    remaining gaps).  The diagonal block, last in every valid row, runs unpipelined steps
//    with the causal mask; while it computes, the next item's Q is loaded into registers
//    (the second score buffer is free then), so its latency is hidden.
//  * Epilogue: O = acc / l rounded to bf16; one exchange between the half-wavefronts
//    (v_permlane32_swap) gives every lane 8 consecutive columns, so each wavefront writes its
//    32 rows with 16-byte stores.
//  * Online softmax ("Block Sparse Attention in LLMs", section 7: tile, never materialise the
//    n x n matrix) in the log2 domain with exp2.  A row's running max is only raised when a
//    step's max exceeds it by more than kRescaleSlack (the final division by the running sum
//    makes the result independent of which max was used), so the O rescale is rare; the
//    decision is per row, so no row's result depends on another row's scores, even in rounding.

#include <atomic>
#include <type_traits>

#include "fwd_common.hpp"

namespace bsa {
namespace {

using namespace fwd;

template <int D, int BLK, int GP, int CK>
struct Cfg {
    static constexpr int NWQ = BLK / 32;              // wavefronts per query head
    static constexpr int NW = NWQ * GP;               // wavefronts per work-group
    static constexpr int NT = NW * 64;                // threads per work-group
    static constexpr int CPT = BLK / CK;              // LDS chunks per key block
    static constexpr int SPC = CK / KC;               // 64-key softmax steps per chunk
    static constexpr int KCH = D / 8;                 // 16-byte chunks per K/V row
    static constexpr int NI = CK * D / 8 / 64;        // 1 KiB direct-to-LDS loads per chunk and tensor
    static constexpr int NI_W = NI / NW;              // ... per wavefront
    static constexpr int KST = 2;                     // K ring stages
    static constexpr int VST = 3;                     // V ring stages (V of a chunk outlives its K)
    static_assert(NI_W * NW == NI, "chunk split");
    static_assert(CPT * CK == BLK && SPC * KC == CK, "chunking");
};

template <bool B>
using flag = std::integral_constant<bool, B>;

template <int D, int BLK, int GP, int CK>
__global__ __launch_bounds__(BLK / 32 * GP * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_bf16_kernel(FwdParams p, int64_t total) {
    using C = Cfg<D, BLK, GP, CK>;
    using Z = Swz<D>;
    __shared__ __attribute__((aligned(1024))) __bf16 sK[C::KST][CK * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV[C::VST][CK * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int g = wv / C::NWQ;  // this wavefront's head within the group
    // 32-row group of the block: the second head takes the groups in reverse order, so that the two
    // wavefronts of a SIMD (wavefronts w and w + NWQ) hold an early and a late group of rows
    const int rg = (GP == 2 && g == 1) ? C::NWQ - 1 - wv % C::NWQ : wv % C::NWQ;
    const int qloc = 32 * rg + l32;  // query row within the block
    const int64_t n = p.n;
    const int hgroups = p.heads_q / GP;
    const int hpk = p.heads_q / p.heads_kv;

    typedef const __attribute__((address_space(4))) int32_t* cptr;  // scalar (uniform) loads
    const cptr rptr = (cptr)p.row_ptr;
    const cptr cidx = (cptr)p.col_idx;

    // ---- work items of this work-group ---------------------------------------------------
    // All item fields are wavefront-uniform 32-bit values (kept in scalar registers).
    struct Item {
        bool ok;
        int i, e0, L;
        int head;     // flattened (batch, query head) of this wavefront
        int kvslice;  // flattened (batch, key/value head)
    };
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    auto item = [&](int k) -> Item {
        Item it{};
        int slice, i;
        it.ok = work_item(blockIdx.x, gridDim.x, k, (int)total, p.nqb, slice, i);
        if (!it.ok) return it;
        const int b = slice / hgroups;
        const int h0 = (slice % hgroups) * GP;
        it.i = uni(i);
        it.head = uni(b * p.heads_q + h0 + g);
        it.kvslice = uni(b * p.heads_kv + h0 / hpk);
        int e0 = rptr[i], e1 = rptr[i + 1];
        e0 = e0 < 0 ? 0 : (e0 > p.nnz ? (int)p.nnz : e0);
        e1 = e1 < e0 ? e0 : (e1 > p.nnz ? (int)p.nnz : e1);
        it.e0 = uni(e0);
        it.L = uni(e1 - e0);
        return it;
    };
    auto kbase = [&](const Item& it) { return (const __bf16*)p.k + (int64_t)it.kvslice * n * D; };
    auto vbase = [&](const Item& it) { return (const __bf16*)p.v + (int64_t)it.kvslice * n * D; };
    // Route entry t of an item; the wavefront-uniform value is taken (and checked) only when
    // the entry is used, a chunk later, so the scalar load never stalls.
    auto col_load = [&](const Item& it, int t) -> int { return cidx[it.e0 + t]; };
    auto col_use = [&](const Item& it, int raw) -> int64_t {
        const int64_t j = __builtin_amdgcn_readfirstlane(raw);
        // A malformed entry (outside [0, i]) is read as block i: every access stays in bounds, and
        // results are defined only for valid routes (bsa_check_route).
        return (j < 0 || j > it.i) ? -1 : j;
    };
    // first global row of chunk `ch` of key block j (an entry outside [0, i] reads block i)
    auto chunk_row = [&](const Item& it, int64_t j, int ch) -> int64_t {
        return (j >= 0 ? j : (int64_t)it.i) * BLK + CK * (ch % C::CPT);
    };

    // ---- asynchronous HBM -> LDS copy of one chunk of CK keys -------------------------------
    // Instruction q of a tensor writes LDS chunks [64q, 64q+64) of the stage, lane-contiguous;
    // each lane fetches the global 16 bytes that the swizzle places there.  Rows past n are
    // clamped to row n-1: they only ever meet masked (future) scores.
    auto issue = [&](const Item& it, int64_t row0, int ks, int vs) {
        // rows are addressed from base row min(row0, n-1) and clamped to row n-1
        const int64_t brow = row0 < n ? row0 : n - 1;
        const int delta = (int)(row0 - brow), last = (int)(n - 1 - brow);
        const char* kb = (const char*)(kbase(it) + brow * D);
        const char* vb = (const char*)(vbase(it) + brow * D);
#pragma unroll
        for (int u = 0; u < C::NI_W; ++u) {
            const int qi = wv * C::NI_W + u;
            const int P = 64 * qi + lane;
            const int r = P / C::KCH, ph = P % C::KCH;
            const int rr = (r + delta) < last ? (r + delta) : last;
            copy16_to_lds(kb, (uint32_t)(rr * D * 2 + ((ph ^ Z::kswz(r)) << 4)), lds_addr(&sK[ks][qi * 512]));
            copy16_to_lds(vb, (uint32_t)(rr * D * 2 + ((ph ^ Z::vswz(r)) << 4)), lds_addr(&sV[vs][qi * 512]));
        }
    };

    // ---- Q fragments (B operand of S^T = K Q^T): Q[row][16kk + 8hf .. +8] ------------------
    bf16x8 qf[D / 16], qn[D / 16];
    auto load_q_into = [&](bf16x8 (&dst)[D / 16], const Item& it) {
        const int64_t qrow = (int64_t)it.i * BLK + qloc;
        const int64_t qr = qrow < n ? qrow : n - 1;
        const __bf16* Qr = (const __bf16*)p.q + ((int64_t)it.head * n + qr) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) dst[kk] = *(const bf16x8*)(Qr + 16 * kk + 8 * hf);
        if (qrow >= n) {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) dst[kk] = bf16x8{};
        }
    };
    auto load_q = [&](const Item& it) {
        const int64_t qrow = (int64_t)it.i * BLK + qloc;
        const int64_t qr = qrow < n ? qrow : n - 1;
        const __bf16* Qr = (const __bf16*)p.q + ((int64_t)it.head * n + qr) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) qf[kk] = *(const bf16x8*)(Qr + 16 * kk + 8 * hf);
        if (qrow >= n) {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) qf[kk] = bf16x8{};
        }
    };

    f32x16 acc[D / 32];
    float m_run, l_run;

    // Per-lane LDS operand offsets (elements).  The swizzles depend only on the row modulo 16,
    // so every operand read is one of these plus a compile-time row offset.
    //  K (A operand of S^T): row l32, logical 16-byte chunk 2kk + hf
    //  V^T (transposing reads): row vr_lane (+8 for the second read), column 32db + vc_lane
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    int kofs[D / 16], vofs[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kofs[kk] = Z::k_off(l32, 2 * kk + hf);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) vofs[db] = Z::v_off(vr_lane, 32 * db + vc_lane);

    // ---- the pieces of one 64-key softmax step ---------------------------------------------
    // S^T[key][query] for keys krow0.. of a K stage (two 32-key accumulators)
    auto s_mma = [&](f32x16 (&sc)[2], const __bf16* Ks, int krow0) {
        sc[0] = f32x16{};
        sc[1] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const bf16x8 a = *(const bf16x8*)(Ks + (krow0 + 32 * c2) * D + kofs[kk]);
                sc[c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sc[c2], 0, 0, 0);
            }
    };
    // causal mask: keys past lim (offset within the step) are invisible to this lane's row
    auto mask = [&](f32x16 (&sc)[2], int lim) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * c2 + 8 * (r >> 2) + 4 * hf + (r & 3);
                if (key > lim) sc[c2][r] = -INFINITY;
            }
    };
    // row max (in-lane, then across the two half-wavefronts) and the lazy rescale
    auto row_max = [&](const f32x16 (&sc)[2]) {
        float mx = -INFINITY;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[c2][r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                         __builtin_bit_cast(uint32_t, mx), false, false);
        return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
    };
    auto rescale = [&](float mx) {
        const float mnew = mx * p.scale_log2;
        const bool need = mnew > m_run + kRescaleSlack;
        if (__any(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
            m_run = need ? mnew : m_run;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
        }
    };
    // P = exp2(s * scale*log2e - m), packed to bf16; row sums of the rounded P
    auto exp_pack = [&](const f32x16 (&sc)[2], uint32_t (&pk)[2][8]) {
        const float mo = (m_run == -INFINITY) ? 0.0f : m_run;  // fully masked so far: weights 0
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[c2][2 * x], p.scale_log2, -mo));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[c2][2 * x + 1], p.scale_log2, -mo));
                pk[c2][x] = pack_bf16x2(p0, p1);
                l_run = dot2_bf16_ones(pk[c2][x], l_run);
            }
    };
    // O^T[d][query] += V^T[d][key] P^T[key][query] over the 64 keys vrow0.. of a V stage
    auto pv = [&](const __bf16* Vs, int vrow0, const uint32_t (&pk)[2][8]) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 bop = __builtin_bit_cast(
                    bf16x8, make_uint4(pk[c2][4 * s], pk[c2][4 * s + 1], pk[c2][4 * s + 2], pk[c2][4 * s + 3]));
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 a = v_fragment_at<D>(Vs + (vrow0 + 32 * c2 + 16 * s) * D + vofs[db]);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[db], 0, 0, 0);
                }
            }
    };

    // ---- persistent loop over this work-group's items ----------------------------------------
    // Chunks stream through the LDS rings across item boundaries (global chunk counter gbase + c:
    // K stage (gbase+c) % 2, V stage (gbase+c) % 3).  The first chunk of the next item is copied
    // during the last chunk of the current one; the current item's O stores drain while the
    // next item computes.
    Item cur = item(0);
    if (!cur.ok) return;
    load_q(cur);
    bool pref = false;  // the current item's first chunk is already in its stages (and landed)
    int gbase = 0;
    f32x16 sA[2], sB[2];
    uint32_t pk[2][8];
    for (int k = 0;; ++k) {
        const Item nxt = item(k + 1);
        const bool nxt_chunks = nxt.ok && nxt.L > 0;
        const int nraw = nxt_chunks ? col_load(nxt, 0) : -1;

#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
        m_run = -INFINITY;
        l_run = 0.f;
        const int L = cur.L;
        const int NCH = L * C::CPT;  // LDS chunks
        if (L > 0) {
            auto kst = [&](int c) { return (gbase + c) & 1; };
            auto vst = [&](int c) { return (gbase + c) % 3; };
            // route window: jA = key block of the current chunk, jB = the next key block
            int64_t jA = col_use(cur, col_load(cur, 0));
            int64_t jB = (L > 1) ? col_use(cur, col_load(cur, 1)) : -1;
            int raw = (L > 2) ? col_load(cur, 2) : -1;
            if (!pref) issue(cur, chunk_row(cur, jA, 0), kst(0), vst(0));

            // B_c: chunk c has landed (this wavefront's copies; the barrier covers the others')
            // and every wavefront is done with the stages that chunk c+1 refills: the K of
            // chunk c-1 (its last scores came before this barrier) and the V of chunk c-2 (its
            // last P V product came before this barrier).  A prefetched first chunk was already
            // awaited before the previous item's stores.
            auto barrier_chunk = [&](int c) {
                if (c > 0 || !pref)
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                else
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (c > 0 && c % C::CPT == 0) {
                    jA = jB;
                    jB = col_use(cur, raw);
                    raw = (c / C::CPT + 2 < L) ? col_load(cur, c / C::CPT + 2) : -1;
                }
                if (c + 1 < NCH)
                    issue(cur, chunk_row(cur, ((c + 1) % C::CPT == 0) ? jB : jA, c + 1), kst(c + 1), vst(c + 1));
                else if (nxt_chunks)
                    issue(nxt, chunk_row(nxt, col_use(nxt, nraw), 0), kst(c + 1), vst(c + 1));
            };
            // causal limit of step place sp of chunk c for this lane's row
            auto limit = [&](int c, int sp) { return jA < 0 ? -1 : qloc - (CK * (c % C::CPT) + KC * sp); };

            // Softmax step t >= 1 of the item (keys [64t, 64t+64) of its chunk stream),
            // software-pipelined and written out in issue order: phase A issues the scores of
            // step t one matrix-core instruction at a time, each followed by the exponentials of
            // one slice of step t-1; phase B issues the P V product of step t-1, each followed by
            // a slice of the row max of step t.  Operands are read from LDS two instructions
            // ahead (a ring of three fragments), and sched_barrier fences keep the compiler from
            // regrouping the slices.  P (the step's parity) names the score buffer; SP is the
            // step's place in its chunk.
            auto iter = [&](int c, auto par, auto place, auto msk) {
                constexpr bool P = decltype(par)::value;
                constexpr int SP = decltype(place)::value;
                constexpr int SPP = (C::SPC == 2) ? 1 - SP : 0;  // place of step t-1
                f32x16(&scur)[2] = P ? sB : sA;
                f32x16(&sprv)[2] = P ? sA : sB;
                constexpr int NMF = D / 8;      // matrix-core instructions per phase
                constexpr int EPM = 16 / NMF;   // exponential pairs per instruction (phase A)
                constexpr int NDB = D / 32;     // 32-wide d blocks of O
                constexpr int MPM = 32 / (NMF - 2) + 1;  // row-max elements per instruction (phase B)

                // ---- phase A: S^T(t) = K Q^T || P(t-1) = exp2(...) ----
                const __bf16* Ks = sK[kst(c)] + KC * SP * D;
                auto kld = [&](int x) {  // A operand of instruction x: keys 32 (x & 1).., d 16 (x >> 1)..
                    return *(const bf16x8*)(Ks + 32 * (x & 1) * D + kofs[x >> 1]);
                };
                const float mo = (m_run == -INFINITY) ? 0.0f : m_run;
                bf16x8 ka[3];
                ka[0] = kld(0);
                ka[1] = kld(1);
                scur[0] = f32x16{};
                scur[1] = f32x16{};
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int x = 0; x < NMF; ++x) {
                    scur[x & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x % 3], qf[x >> 1], scur[x & 1], 0, 0, 0);
                    if (x + 2 < NMF) ka[(x + 2) % 3] = kld(x + 2);
#pragma unroll
                    for (int e = 0; e < EPM; ++e) {
                        const int pr = x * EPM + e;  // pair index 0..15: c2 = pr / 8, word pr % 8
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(sprv[pr >> 3][2 * (pr & 7)], p.scale_log2, -mo));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(sprv[pr >> 3][2 * (pr & 7) + 1], p.scale_log2, -mo));
                        pk[pr >> 3][pr & 7] = pack_bf16x2(p0, p1);
                        l_run = dot2_bf16_ones(pk[pr >> 3][pr & 7], l_run);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (decltype(msk)::value) mask(scur, limit(c, SP));

                // ---- phase B: O^T += V^T P^T(t-1) || row max of S(t) ----
                const __bf16* Vs = sV[vst(SP == 0 ? c - 1 : c)] + KC * SPP * D;
                auto vld = [&](int y) {  // A operand of instruction y: d block y % NDB, keys 16 (y / NDB)..
                    return v_fragment_at<D>(Vs + 16 * (y / NDB) * D + vofs[y % NDB]);
                };
                bf16x8 va[3];
                va[0] = vld(0);
                va[1] = vld(1);
                float mx = -INFINITY;
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int y = 0; y < NMF; ++y) {
                    const int ks = y / NDB;  // 16-key slice: c2 = ks / 2, s = ks % 2
                    const bf16x8 bop = __builtin_bit_cast(
                        bf16x8, make_uint4(pk[ks >> 1][4 * (ks & 1)], pk[ks >> 1][4 * (ks & 1) + 1],
                                           pk[ks >> 1][4 * (ks & 1) + 2], pk[ks >> 1][4 * (ks & 1) + 3]));
                    acc[y % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[y % 3], bop, acc[y % NDB], 0, 0, 0);
                    if (y + 2 < NMF) va[(y + 2) % 3] = vld(y + 2);
                    if (y >= 2) {  // the scores of step t have landed by now
#pragma unroll
                        for (int e = 0; e < MPM; ++e) {
                            const int el = (y - 2) * MPM + e;
                            if (el < 32) mx = fmaxf(mx, scur[el >> 4][el & 15]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                                 __builtin_bit_cast(uint32_t, mx), false, false);
                mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
                rescale(mx);
            };
            using F = flag<false>;
            using T_ = flag<true>;
            using S0 = std::integral_constant<int, 0>;
            using S1 = std::integral_constant<int, 1>;

            // a masked chunk (the diagonal block) runs unpipelined steps in sA
            auto simple_step = [&](int c, int sp) {
                s_mma(sA, sK[kst(c)], KC * sp);
                mask(sA, limit(c, sp));
                rescale(row_max(sA));
                exp_pack(sA, pk);
                pv(sV[vst(c)], KC * sp, pk);
            };
            static_assert((C::CPT == 1 && C::SPC == 2) || (C::SPC == 1 && (C::CPT == 1 || C::CPT == 2)),
                          "a block is one chunk of two steps, or one or two chunks of one step");
            // A valid row lists its key blocks in ascending order and ends with the diagonal
            // block i, so only the chunks of the last block are causally masked; the unmasked
            // chunks run the software pipeline, whose steady state is the only code inside the
            // chunk loop.
            barrier_chunk(0);
            if constexpr (C::SPC == 1) {
                // One softmax step per 64-key chunk, so step c's scores go to sB for odd c and to
                // sA for even c; the loop takes the steps in pairs to keep the buffers
                // compile-time.  Chunks 0 .. NU-1 are unmasked, the last CPT (the diagonal
                // block) masked.
                const int NU = NCH - C::CPT;
                if (NU > 0) {
                    s_mma(sA, sK[kst(0)], 0);
                    rescale(row_max(sA));
                    int c = 1;
                    for (; c + 1 < NU; c += 2) {
                        barrier_chunk(c);
                        iter(c, T_{}, S0{}, F{});
                        barrier_chunk(c + 1);
                        iter(c + 1, F{}, S0{}, F{});
                    }
                    const bool odd_tail = c < NU;  // one unmasked (odd) step left
                    if (odd_tail) {
                        barrier_chunk(c);
                        iter(c, T_{}, S0{}, F{});
                    }
                    barrier_chunk(NU);
                    // finish the pipeline: step NU-1 waits in sB when odd, in sA when even
                    if (odd_tail)
                        exp_pack(sB, pk);
                    else
                        exp_pack(sA, pk);
                    if (nxt.ok) load_q_into(qn, nxt);
                    pv(sV[vst(NU - 1)], 0, pk);
                } else if (nxt.ok) {
                    load_q_into(qn, nxt);
                }
                simple_step(NU, 0);
                if constexpr (C::CPT == 2) {
                    barrier_chunk(NU + 1);
                    simple_step(NU + 1, 0);
                }
            } else if (NCH > 1) {
                s_mma(sA, sK[kst(0)], 0);
                rescale(row_max(sA));
                iter(0, T_{}, S1{}, F{});
                for (int c = 1; c < NCH - 1; ++c) {
                    barrier_chunk(c);
                    // The SIMD arbiter favours the older wavefront (the first head's), which
                    // reaches each barrier first; for the second step of a chunk the second
                    // head's wavefronts take the higher priority, so both arrive together.
                    __builtin_amdgcn_s_setprio(0);
                    iter(c, F{}, S0{}, F{});
                    if (g == 1) __builtin_amdgcn_s_setprio(1);
                    iter(c, T_{}, S1{}, F{});
                }
                __builtin_amdgcn_s_setprio(0);
                barrier_chunk(NCH - 1);
                // finish the pipeline (step (NCH-2, 1) waits in sB)
                exp_pack(sB, pk);
                // the score buffer sB is free until the next item: the next item's Q lands
                // there while the diagonal block computes
                if (nxt.ok) load_q_into(qn, nxt);
                pv(sV[vst(NCH - 2)], KC, pk);
            } else if (nxt.ok) {
                load_q_into(qn, nxt);
            }
            if constexpr (C::SPC == 2) {
                simple_step(NCH - 1, 0);
                // the diagonal block's second step holds keys later than every row of the first
                // KC / 32 row groups: fully masked there, so those wavefronts skip it
                if (32 * rg + 31 >= KC) simple_step(NCH - 1, 1);
            }
            gbase += NCH;
        } else if (nxt.ok) {
            load_q_into(qn, nxt);
        }
        // the next item's first chunk was issued during this item's last chunk; an empty row
        // (malformed route) issued nothing, so the next item copies its first chunk itself
        pref = nxt_chunks && L > 0;
        // this wavefront's copies of the next item's first chunk and its next Q have landed;
        // the stores below are left in flight.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

        // ---- epilogue: O = acc / l, rounded to bf16; optional LSE ------------------------
        const float lt = l_run + __shfl_xor(l_run, 32);
        const float inv = 1.0f / lt;
        const int64_t qrow = (int64_t)cur.i * BLK + qloc;
        if (qrow < n) {
            __bf16* Or = (__bf16*)p.o + ((int64_t)cur.head * n + qrow) * D;
            // A lane holds d = 32 db + 8 j4 + 4 hf + (0..3).  For a pair of j4 (2 jp, 2 jp + 1),
            // one exchange between the half-wavefronts (v_permlane32_swap) gives lane (row, hf)
            // the 8 consecutive d = 32 db + 16 jp + 8 hf + (0..7): one 16-byte store.
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int jp = 0; jp < 2; ++jp) {
                    uint32_t x[2], y[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        x[h] = pack_bf16x2(acc[db][8 * jp + 2 * h] * inv, acc[db][8 * jp + 2 * h + 1] * inv);
                        y[h] = pack_bf16x2(acc[db][8 * jp + 4 + 2 * h] * inv, acc[db][8 * jp + 4 + 2 * h + 1] * inv);
                    }
                    uint32_t lo[2], hi[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(x[h], y[h], false, false);
                        lo[h] = sw[0];  // lanes < 32: own x; lanes >= 32: y of lane - 32
                        hi[h] = sw[1];  // lanes < 32: x of lane + 32; lanes >= 32: own y
                    }
                    *(uint4*)(Or + 32 * db + 16 * jp + 8 * hf) = make_uint4(lo[0], lo[1], hi[0], hi[1]);
                }
            if (p.lse && hf == 0) p.lse[(int64_t)cur.head * n + qrow] = (m_run + __log2f(lt)) * kLn2;
        }
        if (!nxt.ok) break;
        cur = nxt;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) qf[kk] = qn[kk];
    }
}

// Persistent launch: as many work-groups as fit the device at once (queried once per device),
// each walking its share of the work items.
template <int D, int BLK, int GP, int CK>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> resident[kMaxDevices];
    const int64_t total = (int64_t)p.batch * (p.heads_q / GP) * p.nqb;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int slots = (dev >= 0 && dev < kMaxDevices) ? resident[dev].load(std::memory_order_relaxed) : 0;
    if (slots <= 0) {
        int ncu = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fwd_bf16_kernel<D, BLK, GP, CK>,
                                                         Cfg<D, BLK, GP, CK>::NT, 0);
        if (e != hipSuccess) return e;
        slots = (ncu > 0 ? ncu : 1) * (per_cu > 0 ? per_cu : 1);
        if (dev >= 0 && dev < kMaxDevices) resident[dev].store(slots, std::memory_order_relaxed);
    }
    const int64_t grid = total < slots ? total : slots;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BLK, GP, CK>), dim3((unsigned)grid), dim3(Cfg<D, BLK, GP, CK>::NT), 0,
                       stream, p, total);
    return hipGetLastError();
}

}  // namespace

// The pipelined kernel takes 128-token blocks with GQA pairs (one 8-wavefront work-group per
// CU), 64-token blocks with GQA pairs (two 4-wavefront work-groups per CU), and multi-head
// attention over rows longer than about a block and a half (128-token blocks: two 4-wavefront
// work-groups per CU; 64-token blocks: two 2-wavefront ones); the rest goes to the unpipelined
// kernel.
hipError_t launch_fwd_bf16(const FwdParams& p, int d, int block, hipStream_t stream) {
    const int G = p.heads_q / p.heads_kv;
    if (block == 128 && G % 2 == 0) {
        if (d == 64) return launch<64, 128, 2, 128>(p, stream);
        if (d == 128) return launch<128, 128, 2, 128>(p, stream);
    }
    // Multi-head attention at 64-token blocks, rows longer than about a block and a half: two
    // wavefronts per work-group, two work-groups per CU (one wavefront per SIMD); the persistent
    // walk with its copies a chunk ahead still beats one work-group per item on these latency-
    // bound shapes (16 heads, n 4096, d 128: 32.9 -> 27.9 us)
    if (block == 64 && G % 2 != 0 && 2 * p.nnz > 3 * (int64_t)p.nqb) {
        if (d == 64) return launch<64, 64, 1, 64>(p, stream);
        if (d == 128) return launch<128, 64, 1, 64>(p, stream);
    }
    // 64-token blocks with GQA pairs: one 64-key step per chunk, four wavefronts per work-group
    // and 80 KiB of LDS at d = 128, so two work-groups share a CU
    if (block == 64 && G % 2 == 0) {
        if (d == 64) return launch<64, 64, 2, 64>(p, stream);
        if (d == 128) return launch<128, 64, 2, 64>(p, stream);
    }
    // One head per work-group at d = 64: the pipelined kernel pays off once rows hold more than a
    // block or two (it overlaps the next block's copy with the current one); for rows of about
    // one block (the block-diagonal route) the one-item-per-work-group kernel is a little faster
    // (18.0 vs 18.7 us at 2 x 8 heads, n 8192).
    if (block == 128 && d == 64 && 2 * p.nnz > 3 * (int64_t)p.nqb) return launch<64, 128, 1, 128>(p, stream);
    // Multi-head d = 128 at 128-token blocks: 64-key chunks (two per block), so that two
    // 4-wavefront work-groups (80 KiB of LDS each) share a CU
    if (block == 128 && d == 128 && 2 * p.nnz > 3 * (int64_t)p.nqb) return launch<128, 128, 1, 64>(p, stream);
    return launch_fwd_bf16_basic(p, d, block, stream);
}

}  // namespace bsa
