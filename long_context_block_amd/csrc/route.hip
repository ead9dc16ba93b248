// route.hip — integer kernels that write a CSR route (row_ptr, col_idx) on the device.
//
// Route kinds and their sets are documented with bsa_route_kind in bsa.h.  One launch,
// route_build_kernel: one wavefront per query block writes that row's pointer (the closed-form
// start of every row, route_row_start, so no scan is needed) and its key blocks in strictly
// ascending order (self block last).
// Planning is kept apart from the attention kernel, as the BF1 summary times topology
// separately from the sparse kernel ("BF1 ...", section 4 "Kernel and prefill evaluation").

#include "bsa_internal.hpp"

namespace bsa {
namespace {

constexpr int kScanThreads = 1024;

// First SplitMix64 output from state x (golden-ratio increment, then the variant-13 finaliser).
__device__ inline uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline uint64_t pair_hash(uint64_t seed, uint64_t i, uint64_t j) {
    return splitmix64(seed ^ splitmix64((i << 32) | j));
}

// (h, j) lexicographic order
__device__ inline bool key_less(uint64_t ha, int64_t ja, uint64_t hb, int64_t jb) {
    return ha < hb || (ha == hb && ja < jb);
}

__device__ inline uint64_t shfl_xor_u64(uint64_t x, int m) {
    const uint32_t lo = __shfl_xor((uint32_t)x, m);
    const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// One wavefront per query block i (and one for row_ptr[0] when nqb == 0).
__global__ __launch_bounds__(64) void route_build_kernel(bsa_route_spec spec, int64_t nqb,
                                                         int32_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ col_idx) {
    const int64_t i = blockIdx.x;
    const int lane = threadIdx.x;
    if (i == 0 && lane == 0) row_ptr[0] = 0;
    if (i >= nqb) return;
    const int64_t start = route_row_start(spec.kind, i, spec.n_local, spec.keep_first, spec.n_random);
    if (lane == 0)
        row_ptr[i + 1] = (int32_t)(start + route_row_count(spec.kind, i, spec.n_local, spec.keep_first, spec.n_random));
    int32_t* out = col_idx + start;

    if (spec.kind == BSA_ROUTE_BLOCK_DIAGONAL) {
        if (lane == 0) out[0] = (int32_t)i;
        return;
    }
    if (spec.kind == BSA_ROUTE_DENSE_CAUSAL) {
        for (int64_t j = lane; j <= i; j += 64) out[j] = (int32_t)j;
        return;
    }
    if (spec.kind == BSA_ROUTE_SLIDING_WINDOW) {
        const int64_t lo = i > spec.n_local ? i - spec.n_local : 0;
        for (int64_t j = lo + lane; j <= i; j += 64) out[j - lo] = (int32_t)j;
        return;
    }
    if (spec.kind == BSA_ROUTE_BF1) {
        // Merge the descending offset lists {i (block 0)}, {2^k <= i}, {n_local..1} into
        // ascending block indices; the set is O(log i + n_local) long, so one lane does it.
        if (lane != 0) return;
        const int64_t nl = spec.n_local < i ? spec.n_local : i;
        int64_t w = 0;
        int64_t prev = -1;  // last block written
        if (spec.keep_first && i > 0) { out[w++] = 0; prev = 0; }
        int kd = (i > 0) ? floor_log2_u64((uint64_t)i) : -1;  // current dyadic exponent
        int64_t lo = nl;                                     // current local offset
        while (kd >= 0 || lo >= 1) {
            const int64_t od = (kd >= 0) ? ((int64_t)1 << kd) : 0;
            const int64_t off = od > lo ? od : lo;  // largest remaining offset first
            if (od == off) --kd;
            if (lo == off) --lo;
            const int64_t j = i - off;
            if (j > prev) { out[w++] = (int32_t)j; prev = j; }
        }
        out[w] = (int32_t)i;
        return;
    }
    // Static-random: select the m smallest (h, j) keys among the candidates by m rounds of a
    // wavefront-wide minimum over keys strictly above the previous round's minimum, then
    // write the selected blocks in ascending order with a ballot compaction.
    const int64_t c0 = spec.keep_first ? 1 : 0;  // candidates c0 .. i-1
    const int64_t ncand = (i > 0) ? i - c0 : 0;
    const int64_t m = spec.n_random < ncand ? spec.n_random : ncand;
    uint64_t th = ~0ull;  // threshold key (h, j): select keys <= (th, tj)
    int64_t tj = INT64_MAX;
    if (m < ncand) {
        uint64_t ph = 0;
        int64_t pj = -1;  // previous minimum; "no previous" when pj < 0
        for (int64_t r = 0; r < m; ++r) {
            uint64_t bh = ~0ull;
            int64_t bj = INT64_MAX;
            for (int64_t j = c0 + lane; j < i; j += 64) {
                const uint64_t h = pair_hash(spec.seed, (uint64_t)i, (uint64_t)j);
                const bool above = (pj < 0) || key_less(ph, pj, h, j);
                if (above && key_less(h, j, bh, bj)) { bh = h; bj = j; }
            }
            for (int s = 32; s >= 1; s >>= 1) {
                const uint64_t oh = shfl_xor_u64(bh, s);
                const int64_t oj = (int64_t)__shfl_xor((long long)bj, s);
                if (key_less(oh, oj, bh, bj)) { bh = oh; bj = oj; }
            }
            ph = bh;
            pj = bj;
        }
        th = ph;
        tj = pj;
    }
    int64_t w = 0;
    if (spec.keep_first && i > 0) {
        if (lane == 0) out[0] = 0;
        w = 1;
    }
    for (int64_t base = c0; base < i; base += 64) {
        const int64_t j = base + lane;
        bool sel = false;
        if (j < i) {
            if (m == ncand) {
                sel = true;
            } else if (m > 0) {
                const uint64_t h = pair_hash(spec.seed, (uint64_t)i, (uint64_t)j);
                sel = !key_less(th, tj, h, j);  // (h, j) <= threshold
            }
        }
        const uint64_t mask = __ballot(sel);
        const int pos = __popcll(mask & ((1ull << lane) - 1ull));
        if (sel) out[w + pos] = (int32_t)j;
        w += __popcll(mask);
    }
    if (lane == 0) out[w] = (int32_t)i;
}

// ---- transposed route: for key block j, the query blocks i whose row holds j ------------------
// Rows are read as ascending lists (bsa_check_route); membership of j in row i is a binary search.
// Both passes visit i in ascending order, so the output rows are ascending and deterministic.

__device__ inline bool row_holds(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                                 int64_t nnz, int64_t i, int32_t j) {
    int64_t lo = row_ptr[i], hi = row_ptr[i + 1];
    lo = lo < 0 ? 0 : (lo > nnz ? nnz : lo);
    hi = hi < lo ? lo : (hi > nnz ? nnz : hi);
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        const int32_t v = col_idx[mid];
        if (v == j) return true;
        if (v < j) lo = mid + 1; else hi = mid;
    }
    return false;
}

// one wavefront per key block j: t_row_ptr[j + 1] = #{i >= j : j in R(i)}
__global__ __launch_bounds__(64) void route_t_count_kernel(const int32_t* __restrict__ row_ptr,
                                                           const int32_t* __restrict__ col_idx, int64_t nqb,
                                                           int64_t nnz, int32_t* __restrict__ t_row_ptr) {
    const int64_t j = blockIdx.x;
    const int lane = threadIdx.x;
    int cnt = 0;
    for (int64_t i = j + lane; i < nqb; i += 64) cnt += row_holds(row_ptr, col_idx, nnz, i, (int32_t)j) ? 1 : 0;
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) t_row_ptr[j + 1] = cnt;
}

// one work-group: in-place inclusive scan of t_row_ptr[1..nqb]; t_row_ptr[0] = 0.  Every prefix is
// clamped to nnz: rows that overlap (a row_ptr that decreases) can count more memberships than the
// route has entries, and the fill must never write past the caller's nnz-entry t_col_idx.
__global__ __launch_bounds__(kScanThreads) void route_t_scan_kernel(int64_t nqb, int64_t nnz,
                                                                    int32_t* __restrict__ t_row_ptr) {
    __shared__ int64_t part[kScanThreads];
    const int t = threadIdx.x;
    const int64_t per = (nqb + kScanThreads - 1) / kScanThreads;
    const int64_t r0 = t * per;
    const int64_t r1 = (r0 + per < nqb) ? r0 + per : nqb;
    int64_t local = 0;
    for (int64_t x = r0; x < r1; ++x) local += t_row_ptr[x + 1];
    part[t] = local;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int64_t add = (t >= off) ? part[t - off] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    int64_t run = part[t] - local;
    for (int64_t x = r0; x < r1; ++x) {
        run += t_row_ptr[x + 1];
        t_row_ptr[x + 1] = (int32_t)(run < nnz ? run : nnz);
    }
    if (t == 0) t_row_ptr[0] = 0;
}

// one wavefront per key block j: the query blocks i >= j whose row holds j, ascending
__global__ __launch_bounds__(64) void route_t_fill_kernel(const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx, int64_t nqb,
                                                          int64_t nnz, const int32_t* __restrict__ t_row_ptr,
                                                          int32_t* __restrict__ t_col_idx) {
    const int64_t j = blockIdx.x;
    const int lane = threadIdx.x;
    int64_t w = t_row_ptr[j];
    const int64_t end = t_row_ptr[j + 1];
    for (int64_t base = j; base < nqb; base += 64) {
        const int64_t i = base + lane;
        const bool sel = i < nqb && row_holds(row_ptr, col_idx, nnz, i, (int32_t)j);
        const uint64_t mask = __ballot(sel);
        const int pos = __popcll(mask & ((1ull << lane) - 1ull));
        if (sel && w + pos < end && w + pos < nnz) t_col_idx[w + pos] = (int32_t)i;
        w += __popcll(mask);
    }
}

}  // namespace

hipError_t launch_route_transpose(const int32_t* row_ptr, const int32_t* col_idx, int64_t nqb, int64_t nnz,
                                  int32_t* t_row_ptr, int32_t* t_col_idx, hipStream_t stream) {
    if (nqb == 0) {
        hipLaunchKernelGGL(route_t_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, nqb, nnz, t_row_ptr);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(route_t_count_kernel, dim3((unsigned)nqb), dim3(64), 0, stream, row_ptr, col_idx, nqb, nnz,
                       t_row_ptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_t_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, nqb, nnz, t_row_ptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_t_fill_kernel, dim3((unsigned)nqb), dim3(64), 0, stream, row_ptr, col_idx, nqb, nnz,
                       t_row_ptr, t_col_idx);
    return hipGetLastError();
}

hipError_t launch_route_build(const bsa_route_spec& spec, int64_t nqb, int32_t* row_ptr,
                              int32_t* col_idx, hipStream_t stream) {
    hipLaunchKernelGGL(route_build_kernel, dim3((unsigned)(nqb > 0 ? nqb : 1)), dim3(64), 0, stream, spec, nqb,
                       row_ptr, col_idx);
    return hipGetLastError();
}

}  // namespace bsa
