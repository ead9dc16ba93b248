// bwd_dkdv.hip — dK and dV of bfloat16 block-sparse attention on gfx950 matrix cores.
//
// What it computes (the "gradients" correctness gate of "BF1 ...", section 4): for every key t'
// of key/value head g,
//     dV[t'] = sum over (query head h of g, query t with (t, t') selected) of P[t, t'] dO[t],
//     dK[t'] = scale * the same sum of dS[t, t'] Q[t],   dS = P (dP - D),  dP = dO V^T,
// where P = exp(scale q.k - lse) is recomputed from the forward's log-sum-exp, D = rowsum(dO * O)
// (written by bwd_dq_kernel), and a pair takes part when the route selects block (i, j) and, on the
// diagonal block, the query does not precede the key ("Block-Sparse Attention", "Math Or Compute
// Schema").  The sums over t run over the transposed route: the query blocks i whose rows hold j.
//
// How (gfx950):
//  * bwd_dkdv_kernel: one work-group per (batch, key/value head, key block j, segment), 32 keys
//    per wavefront with their K, V rows resident in registers as MFMA B operands.  The segment's
//    work is a run of 64-query units (query block of the transposed row x query head of the group
//    x 64-row part of the block); it is walked in 32-query sub-chunks whose Q and dO rows (plus
//    their log-sum-exp and D) are copied HBM -> LDS (global_load_lds, a ring of NST stages, NST - 1
//    sub-chunks ahead).  Per sub-chunk: S = Q K^T and dP = dO V^T (Q, dO row fragments from LDS),
//    P and dS on the vector unit, then dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read
//    transposed by the LDS unit (ds_read_b64_tr_b16).  Software pipeline: S, dP of sub-chunk
//    t + 1 are issued to the matrix cores one instruction at a time between the exponentials and
//    dS of sub-chunk t.  The accumulation order per accumulator is the plain sequential one.
//    The file is compiled with the MFMA results in VGPRs (--amdgpu-mfma-vgpr-form): dK, dV, S and
//    dP take the 256 architectural VGPRs, and the compiler moves the resident K, V operands (which
//    the matrix cores read from either file) to AGPRs, so the vector unit reads S, dP without
//    copying them out of the accumulation registers first (one wavefront per SIMD either way).
//  * A key block read by many query blocks (block 0 in BF1 is read by all of them) is split into
//    segments of at most kSeg units so that no work-group carries a whole column; a block of one
//    segment stores bf16 dK, dV directly, otherwise each segment writes fp32 partials that
//    bwd_dkdv_reduce_kernel sums in segment order (deterministic, no atomics).

#include "bwd_common.hpp"

namespace bsa {
namespace {

using namespace bwd;

constexpr int kSub = 32;  // queries per sub-chunk
constexpr int NST = 4;    // LDS stages

template <int N>
__device__ inline void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(BwdParams p) {
    constexpr int NW = BLK / 32;
    constexpr int UPB = BLK / kCh;  // 64-query units per query block
    // stage st: tile [st][0] = Q rows, [st][1] = dO rows of one sub-chunk
    __shared__ __attribute__((aligned(1024))) __bf16 sT[NST][2][kSub * D];
    // lse2 of 32 rows, then D; one copy per wavefront, so that all wavefronts issue the same loads
    __shared__ __attribute__((aligned(16))) float sLD[NST][NW][2 * kSub];
    constexpr uint32_t TILE = kSub * D * 2, STAGE = 2 * TILE, LDSTAGE = NW * 2 * kSub * 4;

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bg = blockIdx.x / p.nseg_ub;  // batch * heads_kv + g
    const int sw = (int)(blockIdx.x % p.nseg_ub);
    const int64_t nqb = p.nqb;
    // the segment's descriptor (written by the segment kernel) is read together with the segment
    // count, so the work-group's first dependent load is the sub-chunk table below
    const int4 info = *(const int4*)(p.seg_info + 4 * (int64_t)sw);
    const int nsegs = p.seg_ptr[nqb];
    // (both reads feed the exit test, so they are issued together; a valid descriptor has
    // info.w >= 0, and slots past the segment count hold stale values that are not used)
    if ((sw >= nsegs) | (info.w < 0)) return;
    const int j = info.x;                       // key block
    const int64_t t0 = info.y;                  // its first transposed entry
    const int u_begin = info.z;                 // the segment's first unit
    const int NSUB = info.w & 0xffff;           // its 32-query sub-chunks
    const bool single = (info.w >> 16) & 1;     // the block has one segment
    const int64_t b = bg / p.heads_kv, g = bg % p.heads_kv;
    const int G = p.heads_q / p.heads_kv;
    const int64_t n = p.n, n_pad = p.n_pad;
    const int upt = G * UPB;  // units per entry of the transposed row

    // Sub-chunk table: lane x describes sub-chunks x (index 0) and 64 + x (index 1) by batch *
    // query head, first query row, and kind: the row's offset within the diagonal block
    // (0 .. BLK - 1), BLK off the diagonal, -1 for an entry that is no causal reader of j.
    // Both route reads are issued before the K, V rows below and before any wait (indices
    // clamped to the route, results of lanes past the segment unused).
    static_assert(2 * kSeg <= 128, "two sub-chunks per lane");
    int iqv[2] = {0, 0};
    const int64_t last = p.nnz - 1;
    if (last >= 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int x = 64 * h + lane;
            const int u = u_begin + (x >> 1);
            const int64_t e = t0 + u / upt;
            iqv[h] = p.t_col_idx[e < last ? e : last];
        }
    }

    // this wavefront's 32 keys, resident as B operands: K[key][16kk + 8hf ..], V likewise (rows
    // past n read row 0 and are zeroed)
    const int kloc = 32 * wv + l32;
    const int64_t krow = (int64_t)j * BLK + kloc;
    const bool key_ok = krow < n;
    bf16x8 kf[D / 16], vf[D / 16];
    {
        const __bf16* Kr = (const __bf16*)p.k + (bg * n + (key_ok ? krow : 0)) * D;
        const __bf16* Vr = (const __bf16*)p.v + (bg * n + (key_ok ? krow : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            kf[kk] = *(const bf16x8*)(Kr + 16 * kk + 8 * hf);
            vf[kk] = *(const bf16x8*)(Vr + 16 * kk + 8 * hf);
        }
    }

    int tbh[2], tq0[2], tkind[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int x = 64 * h + lane;
        tbh[h] = 0;
        tq0[h] = 0;
        tkind[h] = -1;
        if (x < NSUB) {
            const int u = u_begin + (x >> 1);
            const int rem = u % upt;
            const int iq = iqv[h];
            const bool bad = iq < j || iq >= nqb;
            const int i = bad ? j : iq;
            tbh[h] = (int)(b * p.heads_q + g * G) + rem / UPB;
            tq0[h] = i * BLK + kCh * (rem % UPB) + kSub * (x & 1);
            tkind[h] = bad ? -1 : (i == j ? tq0[h] - j * BLK : BLK);
        }
    }
    auto fetch = [&](const int(&tab)[2], int x) {
        const int a = __builtin_amdgcn_readlane(tab[0], x & 63), c = __builtin_amdgcn_readlane(tab[1], x & 63);
        return x < 64 ? a : c;
    };
    // Sub-chunks on the diagonal block need the causal mask.  When they form a prefix of the
    // segment (the transposed rows list query blocks in increasing order, so the diagonal entry
    // comes first), only that prefix runs the masked step; otherwise every sub-chunk does.
    int NM;
    {
        const uint64_t m0 = __builtin_amdgcn_ballot_w64(tkind[0] >= 0 && tkind[0] < BLK);
        const uint64_t m1 = __builtin_amdgcn_ballot_w64(tkind[1] >= 0 && tkind[1] < BLK);
        const int c0 = __builtin_popcountll(m0), c1 = __builtin_popcountll(m1);
        auto prefix = [](int c) { return c >= 64 ? ~0ull : ((1ull << c) - 1); };
        const bool pre = (m0 == prefix(c0)) && (c0 == 64 ? m1 == prefix(c1) : m1 == 0);
        NM = pre ? c0 + c1 : NSUB;
    }

    if (!key_ok) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            kf[kk] = bf16x8{};
            vf[kk] = bf16x8{};
        }
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    const uint32_t lds_t = lds_addr(&sT[0][0][0]);
    const uint32_t lds_ld = (uint32_t)(uintptr_t)(const lds_void*)&sLD[0][0];
    // Copy of sub-chunk x into stage st, prepared once and issued in NLD single-instruction
    // parts so that the copies can be spread between matrix-core instructions: the Q tile
    // (NI_W instructions of 64 x 16 bytes per wavefront), the dO tile (NI_W) and the lse2/D run
    // (one dword per lane).  Rows past the head's last row are clamped to it.
    constexpr int NI_W = kSub * D / 512 / NW;
    constexpr int NLD = 2 * NI_W + 1;  // load instructions per copy, the same on every wavefront
    struct Copy {
        const char* qb;
        const char* ob;
        const float* src;
        int delta, lim;
        uint32_t lds, ldl;
    };
    auto prepare = [&](int x, int st) {
        Copy c;
        const int bh = fetch(tbh, x), q0 = fetch(tq0, x), kind = fetch(tkind, x);
        const int64_t r0 = (int64_t)bh * n, row0 = r0 + q0, last = r0 + n - 1;
        const int64_t bse = row0 < last ? row0 : last;
        c.delta = (int)(row0 - bse);
        c.lim = (int)(last - bse);
        c.qb = (const char*)((const __bf16*)p.q + bse * D);
        c.ob = (const char*)((const __bf16*)p.d_o + bse * D);
        c.lds = lds_t + st * STAGE;
        c.ldl = lds_ld + st * LDSTAGE + wv * (2 * kSub * 4);
        // rows q0 .. q0 + 31 < n_pad of the padded lse2 and D, or the pad run (P = 0).  The lane
        // index is re-derived here: a choice between two captured variables would become a load
        // through a chosen pointer and keep both in scratch memory.
        const int ln = threadIdx.x & 63;
        c.src = kind < 0 ? p.ld_pad + ln : (ln >= 32 ? p.dvec : p.lse2) + (int64_t)bh * n_pad + q0 + (ln & 31);
        return c;
    };
    auto issue_part = [&](const Copy& c, int k) {
        if (k < 2 * NI_W) {
            const int qi = wv * NI_W + k % NI_W;
            const int P = 64 * qi + (threadIdx.x & 63);
            const int r = P / Sw2<D>::KCH, pc = P % Sw2<D>::KCH;
            const int rr = (r + c.delta) < c.lim ? (r + c.delta) : c.lim;
            copy16_to_lds(k < NI_W ? c.qb : c.ob, (uint32_t)(rr * D * 2 + ((pc ^ Sw2<D>::f(r)) << 4)),
                          c.lds + (k < NI_W ? 0u : TILE) + 1024u * qi);
        } else {
            issue_dword_at(c.src, c.ldl, 0);
        }
    };
    auto issue = [&](int x, int st) {
        const Copy c = prepare(x, st);
#pragma unroll
        for (int k = 0; k < NLD; ++k) issue_part(c, k);
    };
    // Masked step: pair (query row r of the sub-chunk, this lane's key) takes part when r >= rlo,
    // i.e. on the diagonal block the query does not precede the key; returned minus 4 hf, the
    // lane's accumulator row offset.  Rows past n and excluded entries have lse2 = +inf (P = 0).
    auto row_lo = [&](int x) {
        const int k = fetch(tkind, x);
        return (k >= 0 && k < BLK) ? kloc - k - 4 * hf : -64;
    };
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    constexpr int NMF = D / 8;     // matrix-core instructions per phase (2 x D / 16)
    constexpr int EPM = 16 / NMF;  // score elements (of 16 per lane) per instruction of phase 1
    constexpr int NDB = D / 32;
    static_assert(EPM * NMF == 16 && 2 * NDB * 2 == NMF, "phase shapes");

    // LDS byte addresses of this lane's operand reads in stage 0, tile 0: the row fragments of
    // S, dP (one per 16 columns kk) and the two transposed halves of each 32-column block db.
    // A step adds its stage once per address and hides the sums from the compiler (empty asm),
    // so that tiles and 16-row slices stay constant offsets in the reads' offset field rather
    // than being re-associated into one address register per read.
    uint32_t so[D / 16], to[2 * NDB];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) so[kk] = lds_t + 2 * Sw2<D>::off(l32, 2 * kk + hf);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) to[2 * db + h] = lds_t + 2 * Sw2<D>::toff(vr_lane + 8 * h, 32 * db + vc_lane);
    const uint32_t ldo = lds_ld + wv * (2 * kSub * 4) + 16 * hf;
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
    // S = Q K^T and dP = dO V^T, instruction x: kk = x / 2, x % 2 picks S or dP; sb holds the
    // stage's row-fragment addresses
    auto sc_frag = [&](const uint32_t(&sb)[D / 16], int x) {
        return *(lds_bf16x8*)(uintptr_t)(sb[x >> 1] + (x & 1) * TILE);
    };
    auto stage_bases = [](const auto& src, auto& dst, uint32_t off) {
        constexpr int CNT = sizeof(src) / sizeof(src[0]);
#pragma unroll
        for (int k = 0; k < CNT; ++k) {
            dst[k] = src[k] + off;
            asm volatile("" : "+v"(dst[k]));
        }
    };
    auto sc_mfma = [&](f32x16& s, f32x16& dp, int x, bf16x8 a) {
        if (x & 1)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[x >> 1], dp, 0, 0, 0);
        else
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[x >> 1], s, 0, 0, 0);
    };

    // One step: [S, dP of sub-chunk t + 1 (stage sn)] || [P, dS of sub-chunk t (stage st)], then
    // dV^T += dO^T P, dK^T += Q^T dS of sub-chunk t.  s, dp hold S, dP of t; sn_, dpn receive
    // t + 1.
    constexpr int RING = 4;  // operand fragments in flight: read RING - 1 instructions ahead
    auto step = [&](auto has_next, auto masked, f32x16& s, f32x16& dp, f32x16& sn_, f32x16& dpn, int st, int rlo,
                    const Copy& cp) {
        constexpr bool NEXT = decltype(has_next)::value;
        constexpr bool MASK = decltype(masked)::value;
        const uint32_t so_t = st * STAGE, so_n = (st + 1 < NST ? st + 1 : 0) * STAGE;
        uint32_t lo_t = ldo + st * LDSTAGE;
        asm volatile("" : "+v"(lo_t));
        uint32_t sbn[D / 16], tb[2 * NDB];
        if constexpr (NEXT) stage_bases(so, sbn, so_n);
        stage_bases(to, tb, so_t);
        auto ld_group = [&](int r4, int which) {  // lse2 (0) or D (1) of rows 8 r4 + 4 hf + 0..3
            return *(lds_f32x4*)(uintptr_t)(lo_t + (which * kSub * 4 + r4 * 32));
        };
        uint32_t pp[8], ps[8];
        f32x4 gl[2], gd[2];  // lse2 and D of 4 query rows, one group ahead
        gl[0] = ld_group(0, 0);
        gd[0] = ld_group(0, 1);
        bf16x8 fa[RING];
        if constexpr (NEXT) {
            sn_ = f32x16{};
            dpn = f32x16{};
#pragma unroll
            for (int x = 0; x < RING - 1; ++x) fa[x] = sc_frag(sbn, x);
        }
        float pw[4], dsv[4];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < NMF; ++x) {
            if constexpr (NEXT) {
                sc_mfma(sn_, dpn, x, fa[x % RING]);
                if (x + RING - 1 < NMF) fa[(x + RING - 1) % RING] = sc_frag(sbn, x + RING - 1);
                // the copy of sub-chunk t + 3, one load instruction every few matrix-core ones
#pragma unroll
                for (int k = 0; k < NLD; ++k)
                    if (x == (k * NMF) / NLD + 1) issue_part(cp, k);
            }
#pragma unroll
            for (int u = 0; u < EPM; ++u) {
                const int r = x * EPM + u;  // accumulator element: query row 8 (r / 4) + 4 hf + r % 4
                const int r4 = r >> 2, e = r & 3;
                if (e == 0 && r4 + 1 < 4) {
                    gl[(r4 + 1) & 1] = ld_group(r4 + 1, 0);
                    gd[(r4 + 1) & 1] = ld_group(r4 + 1, 1);
                }
                const float lv = gl[r4 & 1][e], dvv = gd[r4 & 1][e];
                const float ex = __builtin_amdgcn_exp2f(fmaf(s[r], p.scale_log2, -lv));
                if constexpr (MASK)
                    pw[e] = (8 * r4 + e >= rlo) ? ex : 0.f;
                else
                    pw[e] = ex;
                dsv[e] = pw[e] * (dp[r] - dvv);
                if (e & 1) {
                    pp[2 * r4 + (e >> 1)] = pack_bf16x2(pw[e - 1], pw[e]);
                    ps[2 * r4 + (e >> 1)] = pack_bf16x2(dsv[e - 1], dsv[e]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // instruction y: y % 2 picks dV or dK, d block (y / 2) % NDB, 16-query slice y / (2 NDB)
        auto t_frag = [&](int y) {  // dO (y even) or Q (y odd) of stage st, transposed
            const int sl = y / (2 * NDB), db = (y >> 1) % NDB;
            const uint32_t c = ((y & 1) ? 0 : TILE) + sl * 16 * D * 2;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(tb[2 * db] + c));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(tb[2 * db + 1] + c));
            const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
            return __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
        };
        bf16x8 ta[RING];
#pragma unroll
        for (int y = 0; y < RING - 1; ++y) ta[y] = t_frag(y);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int y = 0; y < NMF; ++y) {
            const int sl = y / (2 * NDB), db = (y >> 1) % NDB;
            const uint32_t* src = (y & 1) ? ps : pp;
            const bf16x8 bo = __builtin_bit_cast(
                bf16x8, make_uint4(src[4 * sl], src[4 * sl + 1], src[4 * sl + 2], src[4 * sl + 3]));
            if (y & 1)
                dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[y % RING], bo, dk[db], 0, 0, 0);
            else
                dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[y % RING], bo, dv[db], 0, 0, 0);
            if (y + RING - 1 < NMF) ta[(y + RING - 1) % RING] = t_frag(y + RING - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Pipeline over the segment's sub-chunks t (NSUB is even, so sub-chunks 0 and 1 exist):
    //   step t: [S, dP of t + 1  ||  P, dS of t  ||  copy of t + 3], then dV, dK of t, then wait
    //   for the copy of t + 2 and a barrier.
    // Stage t % NST holds sub-chunk t.  The barrier ending step t makes t + 2 visible to all
    // wavefronts and frees stage t % NST (every wavefront is done with t), which the copy of
    // t + 4 in step t + 1 overwrites.  Copies past the last sub-chunk repeat it into a free stage,
    // so that the number of copies in flight, and with it the wait, stays the same.
    static_assert(NST == 4, "copies run three sub-chunks ahead");
    if (NSUB > 0) {
        auto copy_of = [&](int x) { return prepare(x < NSUB ? x : NSUB - 1, x % NST); };
        issue(0, 0);
        issue(1, 1);
        issue(NSUB > 2 ? 2 : 1, 2);
        wait_vm<NLD>();  // sub-chunks 0 and 1 have landed
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        f32x16 sA, dpA, sB, dpB;
        sA = f32x16{};
        dpA = f32x16{};
#pragma unroll
        for (int x = 0; x < NMF; ++x) sc_mfma(sA, dpA, x, sc_frag(so, x));
        using T_ = std::integral_constant<bool, true>;
        using F_ = std::integral_constant<bool, false>;
        // step t with a successor (t + 1 < NSUB)
        auto body = [&](auto masked, int t, f32x16& s, f32x16& dp, f32x16& sn_, f32x16& dpn) {
            const int rlo = decltype(masked)::value ? row_lo(t) : 0;
            const Copy cp = copy_of(t + 3);
            step(T_{}, masked, s, dp, sn_, dpn, t % NST, rlo, cp);
            wait_vm<NLD>();  // the copy of t + 2 has landed (t + 3 may be in flight)
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        int t = 0;
        for (; t + 2 <= NM && t + 2 < NSUB; t += 2) {  // the diagonal prefix
            body(T_{}, t, sA, dpA, sB, dpB);
            body(T_{}, t + 1, sB, dpB, sA, dpA);
        }
        for (; t + 2 < NSUB; t += 2) {
            body(F_{}, t, sA, dpA, sB, dpB);
            body(F_{}, t + 1, sB, dpB, sA, dpA);
        }
        // t = NSUB - 2: the last two sub-chunks, masked (correct for any sub-chunk)
        body(T_{}, t, sA, dpA, sB, dpB);
        step(F_{}, T_{}, sB, dpB, sA, dpA, (t + 1) % NST, row_lo(t + 1), Copy{});
    }

    // lane holds d = 32 db + 8 j4 + 4 hf + (0..3) of key kloc
    if (single) {
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
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, BLK>), dim3((unsigned)((int64_t)p.batch * p.heads_kv * p.nseg_ub)),
                       dim3(BLK / 32 * 64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<D, BLK>),
                       dim3((unsigned)((int64_t)p.batch * p.heads_kv * p.nqb * (BLK * D / kRedElems))), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdParams& p, int d, int block, hipStream_t stream) {
    if (d == 128) return block == 128 ? launch_t<128, 128>(p, stream) : launch_t<128, 64>(p, stream);
    return block == 128 ? launch_t<64, 128>(p, stream) : launch_t<64, 64>(p, stream);
}

}  // namespace bsa
