// bwd_dkdv.hip — dK and dV of bfloat16 block-sparse attention on gfx950 matrix cores.
//
// What it computes (the "gradients" correctness gate of "BF1 ...", section 4): for every key t'
// of key/value head g,
//     dV[t'] = sum over (query head h of g, query t with (t, t') selected) of P[t, t'] dO[t],
//     dK[t'] = scale * the same sum of dS[t, t'] Q[t],   dS = P (dP - D),  dP = dO V^T,
// where P = exp(scale q.k - lse) is recomputed from the forward's log-sum-exp, D = rowsum(dO * O)
// (bwd_prep_kernel), and a pair takes part when the route selects block (i, j) and, on the
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
//    The file is compiled with the MFMA accumulators allowed in AGPRs: dK, dV (and S, dP) live
//    there, which leaves the 256 architectural VGPRs to K, V, P, dS and the operand rings.
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
constexpr int PD = NST - 1;  // sub-chunks requested ahead of the one in use

template <int N>
__device__ inline void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(BwdParams p) {
    constexpr int NW = BLK / 32;
    constexpr int UPB = BLK / kCh;  // 64-query units per query block
    __shared__ __attribute__((aligned(1024))) __bf16 sQ[NST][kSub * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sO[NST][kSub * D];  // dO
    __shared__ __attribute__((aligned(16))) float sLD[NST][2 * kSub];   // lse of 32 rows, then D

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
    const int units_all = (int)(t1 - t0) * G * UPB;
    const int u_begin = seg * kSeg;
    const int u_end = (u_begin + kSeg < units_all) ? u_begin + kSeg : units_all;
    const int NSUB = u_end > u_begin ? 2 * (u_end - u_begin) : 0;

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

    // sub-chunk x of the segment -> (query block i, batch * query head, first query row)
    auto locate = [&](int x, int64_t& i, int64_t& bh, int64_t& q0) {
        const int u = u_begin + (x >> 1);
        const int ti = u / (G * UPB), rem = u % (G * UPB);
        const int64_t iq = __builtin_amdgcn_readfirstlane(((cptr)p.t_col_idx)[t0 + ti]);
        i = (iq < j || iq >= nqb) ? -1 : iq;  // malformed: a fully masked sub-chunk
        bh = b * p.heads_q + g * G + rem / UPB;
        q0 = (i >= 0 ? i : j) * BLK + kCh * (rem % UPB) + kSub * (x & 1);
    };
    auto issue = [&](int x, int st) {
        int64_t i, bh, q0;
        locate(x, i, bh, q0);
        issue_tile<D, NW, kSub>((const __bf16*)p.q + bh * n * D, q0, n - 1, sQ[st], wv, lane);
        issue_tile<D, NW, kSub>((const __bf16*)p.d_o + bh * n * D, q0, n - 1, sO[st], wv, lane);
        int64_t r = q0 + (lane & 31);
        r = r < n - 1 ? r : n - 1;
        issue_dword((hf ? p.dvec : p.lse) + bh * n + r, sLD[st], wv);
    };
    // load instructions one issue() leaves in flight on this wavefront
    constexpr int PER = 2 * (kSub * D / 512 / NW);
    const int per = PER + (wv == 0 ? 1 : 0);
    // wait until sub-chunk x (issued before the `later` sub-chunks still in flight) has landed
    auto wait_for = [&](int later) {
        if (later >= 2) {
            if (per == PER) wait_vm<2 * PER>(); else wait_vm<2 * (PER + 1)>();
        } else if (later == 1) {
            if (per == PER) wait_vm<PER>(); else wait_vm<PER + 1>();
        } else {
            wait_vm<0>();
        }
    };
    static_assert(PD - 1 <= 2, "wait_for covers up to two later sub-chunks");
    // Pair (query row r of the sub-chunk, this lane's key) takes part when lo <= r < hi: rows
    // past n and, on the diagonal block, queries that precede the key are out; a malformed
    // sub-chunk has hi = 0.  Both bounds are returned minus 4 hf, the lane's accumulator offset.
    auto bounds = [&](int x, int& rlo, int& rhi) {
        int64_t i, bh, q0;
        locate(x, i, bh, q0);
        const int64_t left = n - q0;
        const int hi_ = i < 0 ? 0 : (left < kSub ? (int)left : kSub);
        const int lo_ = (i == j) ? kloc - (int)(q0 - j * BLK) : 0;
        rlo = lo_ - 4 * hf;
        rhi = hi_ - 4 * hf;
    };
    const int vr_lane = 4 * hf + ((lane & 15) >> 2);
    const int vc_lane = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    constexpr int NMF = D / 8;     // matrix-core instructions per phase (2 x D / 16)
    constexpr int EPM = 16 / NMF;  // score elements (of 16 per lane) per instruction of phase 1
    constexpr int NDB = D / 32;
    static_assert(EPM * NMF == 16 && 2 * NDB * 2 == NMF, "phase shapes");

    // S = Q K^T and dP = dO V^T of the sub-chunk in stage st; instruction x: kk = x / 2,
    // x % 2 picks S or dP
    auto sc_frag = [&](int st, int x) { return row_fragment<D>(((x & 1) ? sO : sQ)[st], l32, 2 * (x >> 1) + hf); };
    auto sc_mfma = [&](f32x16& s, f32x16& dp, int x, bf16x8 a) {
        if (x & 1)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[x >> 1], dp, 0, 0, 0);
        else
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[x >> 1], s, 0, 0, 0);
    };

    // One step: [S, dP of sub-chunk t + 1 (stage sn)] || [P, dS of sub-chunk t (stage st)], then
    // dV^T += dO^T P, dK^T += Q^T dS of sub-chunk t.  s, dp hold S, dP of t; sn_, dpn receive t + 1.
    auto step = [&](auto has_next, f32x16& s, f32x16& dp, f32x16& sn_, f32x16& dpn, int st, int sn, int rlo,
                    int rhi) {
        constexpr bool NEXT = decltype(has_next)::value;
        uint32_t pp[8], ps[8];
        float4 gl[2], gd[2];  // log-sum-exp and D of 4 query rows, one group ahead
        gl[0] = *(const float4*)&sLD[st][4 * hf];
        gd[0] = *(const float4*)&sLD[st][kSub + 4 * hf];
        bf16x8 fa[3];
        if constexpr (NEXT) {
            sn_ = f32x16{};
            dpn = f32x16{};
            fa[0] = sc_frag(sn, 0);
            fa[1] = sc_frag(sn, 1);
        }
        float pw[4], dsv[4];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < NMF; ++x) {
            if constexpr (NEXT) {
                sc_mfma(sn_, dpn, x, fa[x % 3]);
                if (x + 2 < NMF) fa[(x + 2) % 3] = sc_frag(sn, x + 2);
            }
#pragma unroll
            for (int u = 0; u < EPM; ++u) {
                const int r = x * EPM + u;  // accumulator element: query row 8 (r / 4) + 4 hf + r % 4
                const int r4 = r >> 2, e = r & 3;
                if (e == 0 && r4 + 1 < 4) {
                    gl[(r4 + 1) & 1] = *(const float4*)&sLD[st][8 * (r4 + 1) + 4 * hf];
                    gd[(r4 + 1) & 1] = *(const float4*)&sLD[st][kSub + 8 * (r4 + 1) + 4 * hf];
                }
                const float4 lq = gl[r4 & 1], dq = gd[r4 & 1];
                const float lv = e == 0 ? lq.x : e == 1 ? lq.y : e == 2 ? lq.z : lq.w;
                const float dvv = e == 0 ? dq.x : e == 1 ? dq.y : e == 2 ? dq.z : dq.w;
                const int rc = 8 * r4 + e;
                const bool ok = rc >= rlo && rc < rhi;
                pw[e] = ok ? __builtin_amdgcn_exp2f(fmaf(s[r], p.scale_log2, -lv * kLog2e)) : 0.f;
                dsv[e] = pw[e] * (dp[r] - dvv);
                if (e & 1) {
                    pp[2 * r4 + (e >> 1)] = pack_bf16x2(pw[e - 1], pw[e]);
                    ps[2 * r4 + (e >> 1)] = pack_bf16x2(dsv[e - 1], dsv[e]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // instruction y: y % 2 picks dV or dK, d block (y / 2) % NDB, 16-query slice y / (2 NDB)
        auto t_frag = [&](int y) {
            const int sl = y / (2 * NDB), db = (y >> 1) % NDB;
            return t_fragment<D>(((y & 1) ? sQ : sO)[st], 16 * sl + vr_lane, 32 * db + vc_lane);
        };
        bf16x8 ta[3];
        ta[0] = t_frag(0);
        ta[1] = t_frag(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int y = 0; y < NMF; ++y) {
            const int sl = y / (2 * NDB), db = (y >> 1) % NDB;
            const uint32_t* src = (y & 1) ? ps : pp;
            const bf16x8 bo = __builtin_bit_cast(
                bf16x8, make_uint4(src[4 * sl], src[4 * sl + 1], src[4 * sl + 2], src[4 * sl + 3]));
            if (y & 1)
                dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[y % 3], bo, dk[db], 0, 0, 0);
            else
                dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[y % 3], bo, dv[db], 0, 0, 0);
            if (y + 2 < NMF) ta[(y + 2) % 3] = t_frag(y + 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (NSUB > 0) {
        // NSUB is even (two sub-chunks per unit), so at least sub-chunks 0 and 1 exist
        for (int x = 0; x < PD && x < NSUB; ++x) issue(x, x);
        wait_for((PD < NSUB ? PD : NSUB) - 1);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        f32x16 sA, dpA, sB, dpB;
        sA = f32x16{};
        dpA = f32x16{};
#pragma unroll
        for (int x = 0; x < NMF; ++x) sc_mfma(sA, dpA, x, sc_frag(0, x));
        int rlo, rhi;
        bounds(0, rlo, rhi);
        using T_ = std::integral_constant<bool, true>;
        using F_ = std::integral_constant<bool, false>;
        // one iteration for sub-chunk t (t + 1 < NSUB): wait for t + 1, request t + PD
        auto body = [&](int t, f32x16& s, f32x16& dp, f32x16& sn_, f32x16& dpn) {
            const int in_flight_last = (t + PD - 1 < NSUB ? t + PD - 1 : NSUB - 1);  // newest requested
            wait_for(in_flight_last - (t + 1));
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (t + PD < NSUB) issue(t + PD, (t + PD) % NST);
            int nlo, nhi;
            bounds(t + 1, nlo, nhi);
            step(T_{}, s, dp, sn_, dpn, t % NST, (t + 1) % NST, rlo, rhi);
            rlo = nlo;
            rhi = nhi;
        };
        int t = 0;
        for (; t + 2 < NSUB; t += 2) {
            body(t, sA, dpA, sB, dpB);
            body(t + 1, sB, dpB, sA, dpA);
        }
        // NSUB even: t = NSUB - 2 here
        body(t, sA, dpA, sB, dpB);
        step(F_{}, sB, dpB, sA, dpA, (t + 1) % NST, 0, rlo, rhi);
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
