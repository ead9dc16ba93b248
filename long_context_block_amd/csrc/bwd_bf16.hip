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
//  * bwd_dq_kernel: one work-group per (batch, query head, query block i), 32 query rows per
//    wavefront.  It first forms D[t] = sum_d dO[t, d] O[t, d] for its rows on the matrix cores
//    (and writes D and lse log2(e) for the dK/dV kernel), then walks row i of the route in 64-key chunks
//    copied HBM -> LDS one chunk ahead (global_load_lds_dwordx4, two stages).  Per chunk, on the matrix cores: S^T = K Q^T and
//    dP^T = V dO^T (K, V rows from LDS; Q, dO resident in registers), then dS^T = P^T (dP^T - D)
//    in registers (one query per lane), then dQ^T += K^T dS^T with K^T read transposed by the
//    LDS unit (ds_read_b64_tr_b16).
//  * dK, dV (bwd_dkdv.hip): the same with the roles of queries and keys exchanged, per key block
//    and segment of its transposed route row; see that file.
//  * Tiles read both row-wise and transposed use one XOR swizzle of 16-byte chunks for both.

#include "bwd_common.hpp"

namespace bsa {
namespace {

using namespace bwd;

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
    // D = rowsum(dO * O) of this lane's row, as the diagonal of the 32 x 32 product O dO^T of
    // the wavefront's rows, formed on the matrix cores with the operand layout and order of
    // dP^T = V dO^T below: where the mathematics makes dP - D vanish (a row whose only selected
    // key is its own token, O = V) it vanishes exactly.  D and lse * log2(e) are also written for
    // the dK/dV kernel, over rows padded to whole blocks (past n: D = 0 and lse2 = +inf, so that a
    // padded query row has P = exp2(s - lse2) = 0 without a mask); this work-group's rows are
    // exactly its block's.
    float dval;
    {
        const __bf16* Or = (const __bf16*)p.o + (bh * n + (row_ok ? qrow : 0)) * D;
        f32x16 x = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const bf16x8 of = row_ok ? *(const bf16x8*)(Or + 16 * kk + 8 * hf) : bf16x8{};
            x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, dof[kk], x, 0, 0, 0);
        }
        // lane l holds column l32 at rows 8 (r / 4) + 4 hf + r % 4: the diagonal entry of column
        // l32 is in the half-wavefront hf = (l32 / 4) % 2, at r = 4 (l32 / 8) + l32 % 4
        const int rd = 4 * (l32 >> 3) + (l32 & 3);
        float mine = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) mine = (r == rd) ? x[r] : mine;
        const float other = __shfl_xor(mine, 32);
        dval = (hf == ((l32 >> 2) & 1)) ? mine : other;
    }
    const float lse2 = row_ok ? p.lse[bh * n + qrow] * kLog2e : 0.f;
    if (hf == 0) {
        p.dvec[bh * p.n_pad + i * BLK + qloc] = dval;
        p.lse2[bh * p.n_pad + i * BLK + qloc] = row_ok ? lse2 : __builtin_inff();
    }
    if (blockIdx.x == 0 && tid < 64) p.ld_pad[tid] = tid < 32 ? __builtin_inff() : 0.f;

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
        // a chunk of the diagonal block whose keys all follow this wavefront's 32 rows adds
        // exactly nothing (P = 0): skipped (the test has one value per wavefront)
        if (j == i && kb > 32 * wv + 31) continue;
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
        // Only the diagonal block (and a malformed entry) has excluded pairs: their scores become
        // -inf in place, so that P = exp2(-inf) = 0 below; a row past n has dO = 0, hence dP = D =
        // 0 and dS = 0, with no mask.
        if (j == i || j < 0) {
            const int lim = (j < 0) ? -1 : qloc - kb;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * c2 + 8 * (r >> 2) + 4 * hf + (r & 3);
                    s[c2][r] = key > lim ? -__builtin_inff() : s[c2][r];
                }
        }
        uint32_t pk[2][8];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                float ds[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * x + e;
                    const float pw = __builtin_amdgcn_exp2f(fmaf(s[c2][r], p.scale_log2, -lse2));
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
    // key block j's first transposed entry a (clamped), its unit count c and its segment count
    auto seg_of = [&](int64_t j, int64_t& a, int64_t& c) -> int64_t {
        a = p.t_row_ptr[j];
        int64_t z = p.t_row_ptr[j + 1];
        a = a < 0 ? 0 : (a > p.nnz ? p.nnz : a);
        z = z < a ? a : (z > p.nnz ? p.nnz : z);
        c = (z - a) * G * cpb;
        const int64_t s = (c + kSeg - 1) / kSeg;
        return s > 1 ? s : 1;
    };
    auto segs = [&](int64_t j) -> int64_t {
        int64_t a, c;
        return seg_of(j, a, c);
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
    // per segment: key block, first transposed entry of the block, first unit, and the segment's
    // 32-query sub-chunk count (at most 2 kSeg) with bit 16 set when the block has one segment;
    // the block's units are dealt evenly over its segments (at most kSeg each)
    for (int64_t j = r0; j < r1; ++j) {
        p.seg_ptr[j] = (int32_t)run;
        int64_t a, c;
        const int64_t sj = seg_of(j, a, c);
        int64_t per = (c + sj - 1) / sj;
        per = per < kSeg ? per : kSeg;
        for (int64_t s = 0; s < sj && run + s < p.nseg_ub; ++s) {
            const int64_t ub = s * per, ue = (ub + per < c) ? ub + per : c;
            const int nsub = ue > ub ? (int)(2 * (ue - ub)) : 0;
            *(int4*)(p.seg_info + 4 * (run + s)) = make_int4((int)j, (int)a, (int)ub, nsub | (sj == 1 ? 1 << 16 : 0));
        }
        run += sj;
    }
    if (t == 1023) p.seg_ptr[nqb] = (int32_t)part[1023];
}

template <int D, int BLK>
hipError_t launch_t(const BwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_seg_kernel, dim3(1), dim3(1024), 0, stream, p, BLK / kCh);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, BLK>), dim3((unsigned)((int64_t)p.batch * p.heads_q * p.nqb)),
                       dim3(BLK / 32 * 64), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_bwd_dkdv(p, D, BLK, stream);
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
