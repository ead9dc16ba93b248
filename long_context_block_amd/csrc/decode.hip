// decode.hip — selected-page decode: one new query token per sequence against the key/value
// blocks ("pages") of its route row.
//
// What it computes ("BF1 ...", section 5 "Selected-page decode characterization"; the
// correctness gate "decode-reference agreement" of section 4): sequence b has seq_lens[b]
// tokens in its key/value cache; its newest token t = seq_lens[b] - 1 sits in query block
// i = floor(t / B) and attends, per query head, to the keys s <= t whose block is in R(i) — the
// row of the same CSR route the prefill uses, built once for the cache capacity (a persistent
// plan).  The result is row t of the prefill output for that token.
//
// How (gfx950).  Decode reads each selected key/value row once and does a few flops per byte, so
// it is bound by memory latency and bandwidth, not by the matrix cores: it runs on the vector
// ALU with coalesced 16-byte loads and no MFMA.
//  * Work is split over 32-key sub-blocks of the row: work unit (b, kv head, group of GC query
//    heads sharing it, split s) takes sub-blocks s, s + S, s + 2S, ... of the row's list, so
//    even batch one spreads the cache read over many compute units.  One wavefront per unit;
//    each key row is read by D*sizeof(T)/16 lanes (16 bytes each), several rows per load.
//  * Per sub-block: scores by per-lane dot products reduced across the lanes of a row, an online
//    softmax in the log2 domain, and the P V product accumulated per lane over its columns.  The
//    unit writes (running max, running sum, unnormalised output) per query head to the
//    caller's workspace.
//  * A second kernel merges the S partials of each (b, query head): the exact softmax merge
//    (rescale every partial to the largest running max), then divides and rounds.

#include "bsa_internal.hpp"
#include "lane_ops.hpp"

namespace bsa {
namespace {

using namespace lanes;

constexpr int kSub = 32;  // keys per sub-block

// element e (0 .. 16/sizeof(T) - 1) of a 16-byte vector of T, as float (bf16 -> fp32 is exact)
template <typename T>
__device__ inline float elem(const uint4& raw, int e) {
    const uint32_t w = e / (4 / sizeof(T)) == 0 ? raw.x : e / (4 / sizeof(T)) == 1 ? raw.y
                     : e / (4 / sizeof(T)) == 2 ? raw.z : raw.w;
    if constexpr (sizeof(T) == 2) return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    return __uint_as_float(w);
}

__device__ inline int64_t clamp_len(int64_t len, int64_t n_max) { return len < 1 ? 1 : (len > n_max ? n_max : len); }

template <typename T, int D, int GC>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeParams p) {
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
    constexpr int LPR = D / VEC;         // lanes per key row
    constexpr int RPI = 64 / LPR;        // key rows per load instruction
    constexpr int NI = kSub / RPI;       // load instructions per sub-block
    static_assert(LPR * VEC == D && RPI * LPR == 64 && NI * RPI == kSub, "lane layout");
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row groups");
    const int lane = threadIdx.x;
    const int r = lane / LPR;  // key row within a load instruction
    const int c = lane % LPR;  // 16-byte column chunk

    int u = blockIdx.x;
    const int s = u % p.splits;
    u /= p.splits;
    const int hc = u % p.hchunks;
    u /= p.hchunks;
    const int g = u % p.heads_kv;
    const int64_t b = u / p.heads_kv;
    const int G = p.heads_q / p.heads_kv;
    const int h0 = g * G + hc * GC;

    const int64_t t = clamp_len(p.seq_lens[b], p.n_max) - 1;
    const int i = (int)(t / p.block);
    const bool csr = p.rkind < 0;
    int e0 = 0, e1 = 0;
    if (csr) {
        e0 = p.row_ptr[i];
        e1 = p.row_ptr[i + 1];
        e0 = e0 < 0 ? 0 : (e0 > p.nnz ? (int)p.nnz : e0);
        e1 = e1 < e0 ? e0 : (e1 > p.nnz ? (int)p.nnz : e1);
    } else {
        e1 = (int)route_row_count(p.rkind, i, p.n_local, p.keep_first, 0);
    }
    const int sh = p.block == 128 ? 2 : 1;  // log2 of the 32-key sub-blocks per block
    const int nsub = (e1 - e0) << sh;

    const T* Kh = (const T*)p.k + (b * p.heads_kv + g) * p.n_max * D + c * VEC;
    const T* Vh = (const T*)p.v + (b * p.heads_kv + g) * p.n_max * D + c * VEC;

    float q[GC][VEC], acc[GC][VEC], m[GC], l[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
        const uint4 qr = *(const uint4*)((const T*)p.q + ((b * p.heads_q + h0 + h) * D + c * VEC));
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            q[h][e] = elem<T>(qr, e) * p.scale_log2;
            acc[h][e] = 0.f;
        }
        m[h] = -INFINITY;
        l[h] = 0.f;
    }

    // first key of the next sub-block of this split at or after sb that holds a selected key
    // (-1: none left); sub-blocks of malformed (non-causal) entries and those wholly past t are
    // skipped
    auto next_sub = [&](int& sb) -> int64_t {
        for (; sb < nsub; sb += p.splits) {
            const int j = csr ? p.col_idx[e0 + (sb >> sh)]
                              : (int)route_row_entry(p.rkind, i, p.n_local, p.keep_first, sb >> sh);
            if (j < 0 || j > i) continue;
            const int64_t k0 = (int64_t)j * p.block + ((sb & ((1 << sh) - 1)) << 5);
            if (k0 <= t) return k0;
        }
        return -1;
    };
    uint4 kf[NI], vf[NI];  // raw 16-byte vectors of the current sub-block, converted on use
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int x = 0; x < NI; ++x) {
            const int64_t key = k0 + x * RPI + r;
            const int64_t kr = key < t ? key : t;  // rows past t are masked; read row t instead
            kf[x] = *(const uint4*)(Kh + kr * D);
            vf[x] = *(const uint4*)(Vh + kr * D);
        }
    };
    int sb = s;
    int64_t k0 = next_sub(sb);
    if (k0 >= 0) load(k0);
    while (k0 >= 0) {
        // the next sub-block's rows are requested before this one is consumed
        int sbn = sb + p.splits;
        const int64_t k1 = next_sub(sbn);
        uint4 kn[NI], vn[NI];
        if (k1 >= 0) {
#pragma unroll
            for (int x = 0; x < NI; ++x) {
                const int64_t key = k1 + x * RPI + r;
                const int64_t kr = key < t ? key : t;
                kn[x] = *(const uint4*)(Kh + kr * D);
                vn[x] = *(const uint4*)(Vh + kr * D);
            }
        }
#pragma unroll
        for (int h = 0; h < GC; ++h) {
            float sc[NI];
            float mx = -INFINITY;
#pragma unroll
            for (int x = 0; x < NI; ++x) {
                float part = 0.f;
#pragma unroll
                for (int e = 0; e < VEC; ++e) part = fmaf(q[h][e], elem<T>(kf[x], e), part);
                part = group_sum<LPR>(part);
                sc[x] = (k0 + x * RPI + r <= t) ? part : -INFINITY;
                mx = fmaxf(mx, sc[x]);
            }
            // max over the row groups (scores are uniform within a group)
            if constexpr (LPR <= 8) mx = fmaxf(mx, xor_lane<8>(mx));
            if constexpr (LPR <= 16) mx = fmaxf(mx, xor_lane<16>(mx));
            mx = fmaxf(mx, xor_lane<32>(mx));
            const float mnew = fmaxf(m[h], mx);  // finite: key k0 <= t is selected
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mnew);
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
#pragma unroll
            for (int x = 0; x < NI; ++x) {
                const float pw = __builtin_amdgcn_exp2f(sc[x] - mnew);
                psum += pw;
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(pw, elem<T>(vf[x], e), acc[h][e]);
            }
            l[h] = l[h] * alpha + psum;
            m[h] = mnew;
        }
        k0 = k1;
        sb = sbn;
#pragma unroll
        for (int x = 0; x < NI; ++x) {
            kf[x] = kn[x];
            vf[x] = vn[x];
        }
    }

    // sum over the key rows held by the different row groups of the wavefront
#pragma unroll
    for (int h = 0; h < GC; ++h) {
        auto across = [&](float x) {
            if constexpr (LPR <= 8) x += xor_lane<8>(x);
            if constexpr (LPR <= 16) x += xor_lane<16>(x);
            return x + xor_lane<32>(x);
        };
        l[h] = across(l[h]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = across(acc[h][e]);
        if (r == 0) {
            float* dst = p.ws + ((b * p.heads_q + h0 + h) * p.splits + s) * (D + 2);
#pragma unroll
            for (int e = 0; e < VEC; ++e) dst[c * VEC + e] = acc[h][e];
            if (c == 0) {
                dst[D] = m[h];
                dst[D + 1] = l[h];
            }
        }
    }
}

// Merge the S partials of one (b, query head): O = sum_s w_s acc_s / sum_s w_s l_s with
// w_s = 2^(m_s - max m); an empty partial (m_s = -inf) has weight 0.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeParams p) {
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    const int S = p.splits;
    const float* base = p.ws + bh * S * (D + 2);
    const float ms = lane < S ? base[lane * (D + 2) + D] : -INFINITY;
    const float ls = lane < S ? base[lane * (D + 2) + D + 1] : 0.f;
    float M = ms;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float w = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    float L = w * ls;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
    const float inv = 1.0f / L;
    // lane = column (D / 64 columns each); the partials are read 16 at a time so that their
    // loads are in flight together
    constexpr int NC = D / 64;
    constexpr int U = 16;
    float o[NC] = {};
    for (int s0 = 0; s0 < S; s0 += U) {
        float a[U][NC], ws[U];
#pragma unroll
        for (int x = 0; x < U; ++x) {
            const int s = s0 + x < S ? s0 + x : S - 1;
            ws[x] = s0 + x < S ? __shfl(w, s) : 0.f;
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) a[x][cc] = base[s * (D + 2) + cc * 64 + lane];
        }
#pragma unroll
        for (int x = 0; x < U; ++x)
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) o[cc] = fmaf(ws[x], a[x][cc], o[cc]);
    }
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
        const int col = cc * 64 + lane;
        const float v = o[cc] * inv;
        if constexpr (sizeof(T) == 2)
            ((__bf16*)p.o)[bh * D + col] = (__bf16)v;  // round to nearest even
        else
            ((float*)p.o)[bh * D + col] = v;
    }
    if (p.lse && lane == 0) p.lse[bh] = (M + __log2f(L)) * 0.69314718055994530942f;
}

template <typename T, int D, int GC>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
    const int64_t units = (int64_t)p.batch * p.heads_kv * p.hchunks * p.splits;
    hipLaunchKernelGGL((decode_partial_kernel<T, D, GC>), dim3((unsigned)units), dim3(64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)((int64_t)p.batch * p.heads_q)), dim3(64), 0,
                       stream, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
    switch (p.gc) {
    case 4: return launch_t<T, D, 4>(p, stream);
    case 2: return launch_t<T, D, 2>(p, stream);
    default: return launch_t<T, D, 1>(p, stream);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t stream) {
    if (bf16) return d == 64 ? launch_d<__bf16, 64>(p, stream) : launch_d<__bf16, 128>(p, stream);
    return d == 64 ? launch_d<float, 64>(p, stream) : launch_d<float, 128>(p, stream);
}

}  // namespace bsa
