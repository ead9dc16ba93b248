// bsa_internal.hpp — declarations shared by the host library and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "bsa.h"

namespace bsa {

// Closed-form |R(i)| for every route kind (see bsa_route_kind in bsa.h for the sets).
// Used by the host (nnz, capacity checks) and by the device route kernels.
__host__ __device__ inline int floor_log2_u64(uint64_t x) { return 63 - __builtin_clzll(x); }
__host__ __device__ inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

__host__ __device__ inline int64_t route_row_count(int kind, int64_t i, int n_local, int keep_first,
                                                   int n_random) {
    switch (kind) {
    case BSA_ROUTE_BF1: {
        if (i == 0) return 1;
        // offsets: local {1..min(n_local,i)} u dyadic {2^k <= i}; offset i is block 0
        const int64_t nl = n_local < i ? n_local : i;
        int64_t offs = nl + floor_log2_u64((uint64_t)i) + 1;
        if (nl >= 1) offs -= floor_log2_u64((uint64_t)nl) + 1;  // powers of two counted twice
        const bool first_already = (i <= n_local) || is_pow2(i);
        return 1 + offs + ((keep_first && !first_already) ? 1 : 0);
    }
    case BSA_ROUTE_BLOCK_DIAGONAL:
        return 1;
    case BSA_ROUTE_DENSE_CAUSAL:
        return i + 1;
    case BSA_ROUTE_STATIC_RANDOM: {
        if (i == 0) return 1;
        const int64_t ncand = keep_first ? i - 1 : i;
        const int64_t m = n_random < ncand ? n_random : ncand;
        return 1 + (keep_first ? 1 : 0) + m;
    }
    case BSA_ROUTE_SLIDING_WINDOW:
        return 1 + (n_local < i ? n_local : i);
    default:
        return -1;
    }
}

// Sum over k = 1 .. m of floor(log2 k) (0 for m <= 0): with K = floor(log2 m), the blocks
// [2^j, 2^(j+1)) for j < K contribute j 2^j each, summing to (K - 2) 2^K + 2, and the partial
// block [2^K, m] contributes K (m - 2^K + 1).
__host__ __device__ inline int64_t sum_floor_log2(int64_t m) {
    if (m <= 0) return 0;
    const int K = floor_log2_u64((uint64_t)m);
    const int64_t p = (int64_t)1 << K;
    return (K - 2) * p + 2 + (int64_t)K * (m - p + 1);
}

// Sum over x = 0 .. N of min(cap, x) (0 for N < 0).
__host__ __device__ inline int64_t sum_min_cap(int64_t N, int64_t cap) {
    if (N < 0) return 0;
    if (N <= cap) return N * (N + 1) / 2;
    return cap * (cap + 1) / 2 + (N - cap) * cap;
}

// Closed-form start of row i in the CSR route: the sum of route_row_count over rows 0 .. i-1
// (row_ptr[i]).  Lets one launch write every row without a scan.
__host__ __device__ inline int64_t route_row_start(int kind, int64_t i, int n_local, int keep_first, int n_random) {
    if (i <= 0) return 0;
    const int64_t kf = keep_first ? 1 : 0;
    switch (kind) {
    case BSA_ROUTE_BF1: {
        // rows r <= n_local hold 0 .. r (r + 1 entries); rows r > n_local hold the self block,
        // n_local local blocks, the dyadic blocks with offset above n_local and, unless r is a
        // power of two, block 0
        const int64_t L = n_local;
        const int64_t A = (i - 1 < L) ? i - 1 : L;  // rows 1 .. A lie inside the window
        int64_t total = 1 + A + A * (A + 1) / 2;    // row 0, then rows 1 .. A
        if (i - 1 > L) {
            const int64_t cnt = i - 1 - L;          // rows L+1 .. i-1
            const int64_t c = L >= 1 ? floor_log2_u64((uint64_t)L) + 1 : 0;  // dyadic offsets <= L
            const int64_t pow2 = (floor_log2_u64((uint64_t)(i - 1)) + 1) - (L >= 1 ? floor_log2_u64((uint64_t)L) + 1 : 0);
            total += cnt * (2 + L - c) + (sum_floor_log2(i - 1) - sum_floor_log2(L)) + kf * (cnt - pow2);
        }
        return total;
    }
    case BSA_ROUTE_BLOCK_DIAGONAL:
        return i;
    case BSA_ROUTE_DENSE_CAUSAL:
        return i * (i + 1) / 2;
    case BSA_ROUTE_STATIC_RANDOM:
        // row 0 holds 1 entry; row r >= 1 holds 1 + kf + min(n_random, r - kf)
        return 1 + (i - 1) * (1 + kf) + sum_min_cap(i - 1 - kf, n_random);
    case BSA_ROUTE_SLIDING_WINDOW:
        return i + sum_min_cap(i - 1, n_local);
    default:
        return -1;
    }
}

// Entry idx (0 <= idx < route_row_count) of row i, ascending, for the routes whose rows have a
// closed form: BF1, block-diagonal, dense causal and sliding window (not static-random, whose
// rows come from a per-row selection).  BF1 with i > n_local lists, in ascending order, block 0
// when keep_first adds it (i not a power of two), the dyadic blocks i - 2^k left of the window
// (2^k > n_local, k from floor(log2 i) down), then the window i - n_local .. i; with i <= n_local
// the window reaches block 0 and the row is 0 .. i.
__host__ __device__ inline int64_t route_row_entry(int kind, int64_t i, int n_local, int keep_first, int64_t idx) {
    switch (kind) {
    case BSA_ROUTE_BLOCK_DIAGONAL:
        return i;
    case BSA_ROUTE_DENSE_CAUSAL:
        return idx;
    case BSA_ROUTE_SLIDING_WINDOW:
        return (i > n_local ? i - n_local : 0) + idx;
    case BSA_ROUTE_BF1: {
        if (i <= n_local) return idx;
        if (keep_first && !is_pow2(i)) {
            if (idx == 0) return 0;
            --idx;
        }
        const int kmax = floor_log2_u64((uint64_t)i);
        const int kmin = n_local == 0 ? 0 : floor_log2_u64((uint64_t)n_local) + 1;  // 2^kmin > n_local
        const int64_t nd = kmax >= kmin ? kmax - kmin + 1 : 0;
        if (idx < nd) return i - ((int64_t)1 << (kmax - idx));
        return i - n_local + (idx - nd);
    }
    default:
        return -1;
    }
}

// Launchers (defined in the kernel translation units).  They only enqueue work and return
// the hipError_t of the launch.
hipError_t launch_route_build(const bsa_route_spec& spec, int64_t nqb, int32_t* row_ptr,
                              int32_t* col_idx, hipStream_t stream);
hipError_t launch_route_transpose(const int32_t* row_ptr, const int32_t* col_idx, int64_t nqb, int64_t nnz,
                                  int32_t* t_row_ptr, int32_t* t_col_idx, hipStream_t stream);

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    int32_t batch, heads_q, heads_kv;
    int32_t nqb;
    int64_t n;
    int64_t nnz;
    float scale_log2;  // softmax scale * log2(e): scores are exponentiated with exp2
};

struct DecodeParams {
    const void* q;  // [batch, heads_q, d]
    const void* k;  // [batch, heads_kv, n_max, d]
    const void* v;
    void* o;        // [batch, heads_q, d]
    float* lse;     // [batch, heads_q] or null
    const int32_t* seq_lens;
    const int32_t* row_ptr;  // CSR route (rkind < 0)
    const int32_t* col_idx;
    float* ws;      // [batch, heads_q, splits, d + 2] partials
    int32_t rkind;  // < 0: rows from row_ptr/col_idx; else a closed-form bsa_route_kind
    int32_t n_local, keep_first;
    int32_t batch, heads_q, heads_kv, block;
    int32_t splits;   // split units per (b, kv head, head group), <= kDecodeMaxSplits
    int32_t hchunks;  // query-head groups per kv head
    int32_t gc;       // query heads per group (1, 2, 4)
    int64_t n_max;
    int64_t nnz;
    float scale_log2;
};
constexpr int kDecodeMaxSplits = 64;

struct BwdParams {
    const void* q;    // [batch, heads_q, n, d]
    const void* k;    // [batch, heads_kv, n, d]
    const void* v;
    const void* o;    // forward output
    const void* d_o;  // upstream gradient of o
    const float* lse; // forward log-sum-exp (natural log) [batch, heads_q, n]
    void* dq;
    void* dk;
    void* dv;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const int32_t* t_row_ptr;  // transposed route: query blocks reading key block j
    const int32_t* t_col_idx;
    float* dvec;      // workspace: D = rowsum(dO * O) [batch, heads_q, n_pad], 0 past n
    float* lse2;      // workspace: lse * log2(e) [batch, heads_q, n_pad], +inf past n
    float* ld_pad;    // workspace: 32 x +inf, then 32 x 0: lse2 and D of a fully excluded row run
    int32_t* seg_ptr; // workspace: [nqb + 1] segment prefix of the transposed rows
    int32_t* seg_info;// workspace: [nseg_ub, 4] per segment: key block, its first transposed entry, the segment's
                      // first unit, its sub-chunk count (| 1 << 16 when the block has one segment)
    float* part;      // workspace: [batch * heads_kv * nseg_ub, 2, block, d] partial dK, dV
    int32_t batch, heads_q, heads_kv;
    int32_t nqb;
    int64_t n;
    int64_t n_pad;    // n rounded up to a whole block
    int64_t nnz;
    int64_t nseg_ub;  // segments per (batch, kv head), upper bound
    float scale;
    float scale_log2;
};

struct BsbrParams {
    const void* q;    // [batch, heads_q, n, d] bf16
    const void* k;    // [batch, heads_kv, n, d]
    const void* v;
    const void* r;    // meta queries [batch, heads_q, nch, d]
    const void* h;    // meta keys [batch, heads_kv, nch, d]
    void* o;          // [batch, heads_q, n, d]
    float* F;         // workspace: chunk states [batch, heads_kv, nch, d * d] (32 x 32 tiles)
    float* A;         // workspace: retrieved states [batch, heads_q, nch, d * d]
    int32_t batch, heads_q, heads_kv, nch;
    int64_t n;
    float scale_log2;
};
hipError_t launch_bsbr(const BsbrParams& p, int d, int chunk, hipStream_t stream);

int64_t bwd_segments_upper_bound(int64_t nqb, int64_t nnz, int heads_q, int heads_kv, int block);
hipError_t launch_bwd_bf16(const BwdParams& p, int d, int block, hipStream_t stream);

hipError_t launch_fwd_bf16(const FwdParams& p, int d, int block, hipStream_t stream);

// Device address of the current device's copy of the library's static scratch array
// (BSA_STATIC_SCRATCH_BYTES), looked up once per device (static_scratch.hip).
hipError_t static_scratch(void** ptr);
hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t stream);
hipError_t launch_fwd_bf16_basic(const FwdParams& p, int d, int block, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int d, int block, hipStream_t stream);

}  // namespace bsa
