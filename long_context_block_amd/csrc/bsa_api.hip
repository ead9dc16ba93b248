// bsa_api.hip — the C ABI of libbsa.so: argument validation, dispatch, error reporting.
//
// Every argument is validated on the host before any HIP call, so invalid calls do no device
// work and are testable without a GPU.  Nothing is allocated; all device work goes onto the
// caller's stream.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "bsa_internal.hpp"

namespace {

thread_local std::string g_last_error;

bsa_status fail(bsa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bsa_status ok() {
    g_last_error.clear();
    return BSA_OK;
}

bsa_status device_error(hipError_t e, const char* where) {
    return fail(BSA_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Host-side nnz of a route: the closed-form start of the row past the last one (the same
// function the route kernel writes row_ptr with); -1 if it does not fit int32.
int64_t route_nnz(const bsa_route_spec& s, int64_t nqb) {
    const int64_t total = bsa::route_row_start(s.kind, nqb, s.n_local, s.keep_first, s.n_random);
    return (total < 0 || total > INT32_MAX) ? -1 : total;
}

bsa_status check_route_host(const int32_t* rp, const int32_t* ci, int64_t nqb, int64_t nnz) {
    if (rp[0] != 0) return fail(BSA_ERR_BAD_ROUTE, "row_ptr[0] = %d, expected 0", rp[0]);
    if ((int64_t)rp[nqb] != nnz)
        return fail(BSA_ERR_BAD_ROUTE, "row_ptr[nqb] = %d, expected nnz = %lld", rp[nqb], (long long)nnz);
    for (int64_t i = 0; i < nqb; ++i) {
        const int64_t a = rp[i], b = rp[i + 1];
        if (b < a) return fail(BSA_ERR_BAD_ROUTE, "row_ptr decreases at row %lld", (long long)i);
        if (b == a) return fail(BSA_ERR_BAD_ROUTE, "row %lld is empty (the self block is mandatory)", (long long)i);
        for (int64_t e = a; e < b; ++e) {
            const int64_t j = ci[e];
            if (j < 0 || j > i)
                return fail(BSA_ERR_BAD_ROUTE, "row %lld reads block %lld outside [0, %lld]", (long long)i,
                            (long long)j, (long long)i);
            if (e > a && j <= ci[e - 1])
                return fail(BSA_ERR_BAD_ROUTE, "row %lld is not strictly ascending", (long long)i);
        }
        if (ci[b - 1] != i) return fail(BSA_ERR_BAD_ROUTE, "row %lld does not end with its own block", (long long)i);
    }
    return ok();
}

bsa_status validate_forward(const void* q, const void* k, const void* v, void* o, const float* lse,
                            int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d,
                            int32_t block, bsa_dtype dtype, const int32_t* row_ptr,
                            const int32_t* col_idx, int64_t nnz, bool check_nnz) {
    if (batch < 0 || heads_q < 1 || heads_kv < 1 || n < 0 || block < 1 || d < 1)
        return fail(BSA_ERR_INVALID_ARGUMENT,
                    "sizes must satisfy batch >= 0, heads >= 1, n >= 0, d >= 1, block >= 1 "
                    "(got batch=%d heads_q=%d heads_kv=%d n=%lld d=%d block=%d)",
                    batch, heads_q, heads_kv, (long long)n, d, block);
    if (heads_q % heads_kv != 0)
        return fail(BSA_ERR_INVALID_ARGUMENT, "heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
    if (dtype != BSA_BF16 && dtype != BSA_FP32) return fail(BSA_ERR_UNSUPPORTED, "dtype %d not supported", (int)dtype);
    if (d != 64 && d != 128) return fail(BSA_ERR_UNSUPPORTED, "head dim d=%d not supported (64 or 128)", d);
    if (block != 64 && block != 128) return fail(BSA_ERR_UNSUPPORTED, "block=%d not supported (64 or 128)", block);
    const int64_t nqb = (n + block - 1) / block;
    if (nqb > INT32_MAX - 1) return fail(BSA_ERR_UNSUPPORTED, "too many blocks (%lld)", (long long)nqb);
    if (batch == 0 || n == 0) return ok();
    if (!q || !k || !v || !o) return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v and o must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v and o must be 16-byte aligned");
    if (lse && ((uintptr_t)lse & 3u)) return fail(BSA_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    if (check_nnz) {
        if (!row_ptr || !col_idx) return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr and col_idx must be non-NULL");
        if (nnz < nqb || nnz > INT32_MAX)
            return fail(BSA_ERR_INVALID_ARGUMENT, "nnz=%lld must be in [nqb=%lld, 2^31)", (long long)nnz, (long long)nqb);
    }
    const int G = heads_q / heads_kv;
    const int gp = (dtype == BSA_BF16 && G % 2 == 0) ? 2 : 1;
    const int64_t wg = (int64_t)batch * (heads_q / gp) * nqb * (dtype == BSA_FP32 ? (block + 15) / 16 : 1);
    if (wg > INT32_MAX) return fail(BSA_ERR_UNSUPPORTED, "grid of %lld work-groups too large", (long long)wg);
    return ok();
}

bool env_validate_route() {
    const char* s = getenv("BSA_VALIDATE_ROUTE");
    return s && s[0] && strcmp(s, "0") != 0;
}

bsa_status run_forward(const void* q, const void* k, const void* v, void* o, float* lse, int32_t batch,
                       int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d, int32_t block,
                       bsa_dtype dtype, float scale, const int32_t* row_ptr, const int32_t* col_idx,
                       int64_t nnz, hipStream_t stream) {
    bsa::FwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.row_ptr = row_ptr; p.col_idx = col_idx;
    p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv;
    p.nqb = (int32_t)((n + block - 1) / block);
    p.n = n;
    p.nnz = nnz;
    const double sc = (scale > 0.f) ? (double)scale : 1.0 / std::sqrt((double)d);
    p.scale_log2 = (float)(sc * 1.4426950408889634073599);
    const hipError_t e = (dtype == BSA_BF16) ? bsa::launch_fwd_bf16(p, d, block, stream)
                                             : bsa::launch_fwd_f32(p, d, block, stream);
    if (e != hipSuccess) return device_error(e, "forward launch");
    return ok();
}

}  // namespace

extern "C" {

const char* bsa_status_string(bsa_status s) {
    switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARGUMENT: return "BSA_ERR_INVALID_ARGUMENT";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_BAD_ROUTE: return "BSA_ERR_BAD_ROUTE";
    case BSA_ERR_CAPACITY: return "BSA_ERR_CAPACITY";
    case BSA_ERR_DEVICE: return "BSA_ERR_DEVICE";
    }
    return "BSA_ERR_UNKNOWN";
}

const char* bsa_last_error(void) { return g_last_error.c_str(); }

bsa_status bsa_check_route(const int32_t* row_ptr, const int32_t* col_idx, int64_t nqb, int64_t nnz) {
    if (nqb < 0 || nnz < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "nqb and nnz must be >= 0");
    if (!row_ptr) return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr must be non-NULL");
    if (nnz > 0 && !col_idx) return fail(BSA_ERR_INVALID_ARGUMENT, "col_idx must be non-NULL");
    return check_route_host(row_ptr, col_idx, nqb, nnz);
}

bsa_status bsa_build_route(const bsa_route_spec* spec, int64_t n, int32_t block, int32_t* row_ptr,
                           int32_t* col_idx, int64_t col_capacity, int64_t* nnz_out, hipStream_t stream) {
    if (!spec || !nnz_out) return fail(BSA_ERR_INVALID_ARGUMENT, "spec and nnz_out must be non-NULL");
    if (n < 0 || block < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "need n >= 0 and block >= 1");
    if (spec->kind < BSA_ROUTE_BF1 || spec->kind > BSA_ROUTE_SLIDING_WINDOW)
        return fail(BSA_ERR_INVALID_ARGUMENT, "unknown route kind %d", spec->kind);
    if (spec->n_local < 0 || spec->n_random < 0)
        return fail(BSA_ERR_INVALID_ARGUMENT, "n_local and n_random must be >= 0");
    const int64_t nqb = (n + block - 1) / block;
    if (nqb > INT32_MAX - 1) return fail(BSA_ERR_UNSUPPORTED, "too many blocks (%lld)", (long long)nqb);
    if (spec->kind == BSA_ROUTE_DENSE_CAUSAL && nqb > 65535)
        return fail(BSA_ERR_UNSUPPORTED, "dense route with %lld blocks exceeds 2^31 entries", (long long)nqb);
    const int64_t nnz = route_nnz(*spec, nqb);
    if (nnz < 0) return fail(BSA_ERR_UNSUPPORTED, "route has 2^31 or more entries");
    *nnz_out = nnz;
    if (!row_ptr) return ok();  // size query
    if (!col_idx && nnz > 0) return fail(BSA_ERR_INVALID_ARGUMENT, "col_idx must be non-NULL when nnz > 0");
    if (col_capacity < nnz)
        return fail(BSA_ERR_CAPACITY, "col_capacity %lld < nnz %lld", (long long)col_capacity, (long long)nnz);
    const hipError_t e = bsa::launch_route_build(*spec, nqb, row_ptr, col_idx, stream);
    if (e != hipSuccess) return device_error(e, "route build launch");
    return ok();
}

bsa_status bsa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int32_t batch,
                       int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d, int32_t block,
                       bsa_dtype dtype, float scale, const int32_t* row_ptr, const int32_t* col_idx,
                       int64_t nnz, hipStream_t stream) {
    bsa_status s = validate_forward(q, k, v, o, lse, batch, heads_q, heads_kv, n, d, block, dtype, row_ptr,
                                    col_idx, nnz, true);
    if (s != BSA_OK || batch == 0 || n == 0) return s;
    if (!(scale <= 0.f) && !std::isfinite(scale))
        return fail(BSA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (env_validate_route()) {
        const int64_t nqb = (n + block - 1) / block;
        std::vector<int32_t> rp(nqb + 1), ci(nnz);
        hipError_t e = hipMemcpyAsync(rp.data(), row_ptr, rp.size() * 4, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipMemcpyAsync(ci.data(), col_idx, ci.size() * 4, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return device_error(e, "route validation copy");
        s = check_route_host(rp.data(), ci.data(), nqb, nnz);
        if (s != BSA_OK) return s;
    }
    return run_forward(q, k, v, o, lse, batch, heads_q, heads_kv, n, d, block, dtype, scale, row_ptr, col_idx,
                       nnz, stream);
}

bsa_status bsa_build_route_transpose(const int32_t* row_ptr, const int32_t* col_idx, int64_t nqb, int64_t nnz,
                                     int32_t* t_row_ptr, int32_t* t_col_idx, hipStream_t stream) {
    if (nqb < 0 || nnz < 0 || nnz > INT32_MAX || nqb > INT32_MAX - 1)
        return fail(BSA_ERR_INVALID_ARGUMENT, "need 0 <= nqb < 2^31 - 1 and 0 <= nnz < 2^31");
    if (!row_ptr || !t_row_ptr) return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr and t_row_ptr must be non-NULL");
    if (nnz > 0 && (!col_idx || !t_col_idx))
        return fail(BSA_ERR_INVALID_ARGUMENT, "col_idx and t_col_idx must be non-NULL when nnz > 0");
    const hipError_t e = bsa::launch_route_transpose(row_ptr, col_idx, nqb, nnz, t_row_ptr, t_col_idx, stream);
    if (e != hipSuccess) return device_error(e, "route transpose launch");
    return ok();
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}

size_t bsa_backward_workspace_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d,
                                    int32_t block, int64_t nnz) {
    if (batch < 0 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv || n < 0 || d < 1 || block < 64 || nnz < 0)
        return 0;
    const int64_t nqb = (n + block - 1) / block;
    const int64_t segs = bsa::bwd_segments_upper_bound(nqb, nnz, heads_q, heads_kv, block);
    return align256((size_t)2 * batch * heads_q * nqb * block * sizeof(float)) + 256 +
           align256((size_t)(nqb + 1) * sizeof(int32_t)) + align256((size_t)segs * 4 * sizeof(int32_t)) +
           (size_t)batch * heads_kv * segs * 2 * block * d * sizeof(float);
}

bsa_status bsa_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                        void* dq, void* dk, void* dv, int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n,
                        int32_t d, int32_t block, bsa_dtype dtype, float scale, const int32_t* row_ptr,
                        const int32_t* col_idx, int64_t nnz, const int32_t* t_row_ptr, const int32_t* t_col_idx,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    bsa_status s = validate_forward(q, k, v, dq, nullptr, batch, heads_q, heads_kv, n, d, block, dtype, row_ptr,
                                    col_idx, nnz, true);
    if (s != BSA_OK) return s;
    if (dtype != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "the backward supports bf16 only");
    if (!(scale <= 0.f) && !std::isfinite(scale)) return fail(BSA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (batch == 0 || n == 0) return ok();
    if (!o || !d_o || !lse || !dk || !dv || !t_row_ptr || !t_col_idx || !workspace)
        return fail(BSA_ERR_INVALID_ARGUMENT, "o, d_o, lse, dk, dv, the transposed route and workspace must be non-NULL");
    if (!aligned16(o) || !aligned16(d_o) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return fail(BSA_ERR_INVALID_ARGUMENT, "o, d_o, dk, dv and workspace must be 16-byte aligned");
    if (((uintptr_t)lse & 3u) != 0) return fail(BSA_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    const size_t need = bsa_backward_workspace_bytes(batch, heads_q, heads_kv, n, d, block, nnz);
    if (workspace_bytes < need) return fail(BSA_ERR_CAPACITY, "workspace_bytes %zu < %zu", workspace_bytes, need);
    const int64_t nqb = (n + block - 1) / block;
    const int64_t segs = bsa::bwd_segments_upper_bound(nqb, nnz, heads_q, heads_kv, block);
    if (nqb * block > INT32_MAX) return fail(BSA_ERR_UNSUPPORTED, "n=%lld too large for the backward", (long long)n);
    if ((int64_t)batch * heads_kv * segs > INT32_MAX || (int64_t)batch * heads_q * nqb > INT32_MAX ||
        (int64_t)batch * heads_kv * nqb * 16 > INT32_MAX)
        return fail(BSA_ERR_UNSUPPORTED, "grid too large");
    bsa::BwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.d_o = d_o; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.row_ptr = row_ptr; p.col_idx = col_idx; p.t_row_ptr = t_row_ptr; p.t_col_idx = t_col_idx;
    char* ws = (char*)workspace;
    const int64_t n_pad = nqb * block;
    p.dvec = (float*)ws;
    p.lse2 = p.dvec + (size_t)batch * heads_q * n_pad;
    ws += align256((size_t)2 * batch * heads_q * n_pad * sizeof(float));
    p.ld_pad = (float*)ws;
    ws += 256;
    p.seg_ptr = (int32_t*)ws;
    ws += align256((size_t)(nqb + 1) * sizeof(int32_t));
    p.seg_info = (int32_t*)ws;
    ws += align256((size_t)segs * 4 * sizeof(int32_t));
    p.part = (float*)ws;
    p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv;
    p.nqb = (int32_t)nqb; p.n = n; p.n_pad = n_pad; p.nnz = nnz; p.nseg_ub = segs;
    const double sc = (scale > 0.f) ? (double)scale : 1.0 / std::sqrt((double)d);
    p.scale = (float)sc;
    p.scale_log2 = (float)(sc * 1.4426950408889634073599);
    const hipError_t e = bsa::launch_bwd_bf16(p, d, block, stream);
    if (e != hipSuccess) return device_error(e, "backward launch");
    return ok();
}

size_t bsa_decode_workspace_bytes(int32_t batch, int32_t heads_q, int32_t d) {
    if (batch < 0 || heads_q < 1 || d < 1) return 0;
    return (size_t)batch * heads_q * bsa::kDecodeMaxSplits * (d + 2) * sizeof(float);
}

namespace {

// Shared by bsa_decode (CSR route: row_ptr/col_idx/nnz), bsa_decode_routed (spec) and
// bsa_decode_routed_noalloc (spec, the library's static scratch array: static_ws).
bsa_status decode_impl(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                       const int32_t* seq_lens, int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n_max,
                       int32_t d, int32_t block, bsa_dtype dtype, float scale, const int32_t* row_ptr,
                       const int32_t* col_idx, int64_t nnz, const bsa_route_spec* spec, float* workspace,
                       size_t workspace_bytes, hipStream_t stream, bool static_ws = false) {
    if (batch < 0 || heads_q < 1 || heads_kv < 1 || n_max < 1 || block < 1 || d < 1)
        return fail(BSA_ERR_INVALID_ARGUMENT,
                    "sizes must satisfy batch >= 0, heads >= 1, n_max >= 1, d >= 1, block >= 1 "
                    "(got batch=%d heads_q=%d heads_kv=%d n_max=%lld d=%d block=%d)",
                    batch, heads_q, heads_kv, (long long)n_max, d, block);
    if (heads_q % heads_kv != 0)
        return fail(BSA_ERR_INVALID_ARGUMENT, "heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
    if (dtype != BSA_BF16 && dtype != BSA_FP32) return fail(BSA_ERR_UNSUPPORTED, "dtype %d not supported", (int)dtype);
    if (d != 64 && d != 128) return fail(BSA_ERR_UNSUPPORTED, "head dim d=%d not supported (64 or 128)", d);
    if (block != 64 && block != 128) return fail(BSA_ERR_UNSUPPORTED, "block=%d not supported (64 or 128)", block);
    if (!(scale <= 0.f) && !std::isfinite(scale)) return fail(BSA_ERR_INVALID_ARGUMENT, "scale must be finite");
    const int64_t nqb = (n_max + block - 1) / block;
    if (nqb > INT32_MAX - 1) return fail(BSA_ERR_UNSUPPORTED, "too many blocks (%lld)", (long long)nqb);
    if (spec) {
        if (spec->kind < BSA_ROUTE_BF1 || spec->kind > BSA_ROUTE_SLIDING_WINDOW)
            return fail(BSA_ERR_INVALID_ARGUMENT, "unknown route kind %d", spec->kind);
        if (spec->kind == BSA_ROUTE_STATIC_RANDOM)
            return fail(BSA_ERR_UNSUPPORTED, "static-random rows have no closed form: build the route and use bsa_decode");
        if (spec->n_local < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "n_local must be >= 0");
    }
    if (batch == 0) return ok();
    if (!q || !k_cache || !v_cache || !o || !seq_lens || (!static_ws && !workspace) || (!spec && (!row_ptr || !col_idx)))
        return fail(BSA_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache, o, seq_lens, route and workspace must be non-NULL");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        (!static_ws && !aligned16(workspace)))
        return fail(BSA_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache, o and workspace must be 16-byte aligned");
    if (lse && ((uintptr_t)lse & 3u)) return fail(BSA_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    if (((uintptr_t)seq_lens & 3u) != 0) return fail(BSA_ERR_INVALID_ARGUMENT, "seq_lens must be 4-byte aligned");
    if (!spec && (nnz < nqb || nnz > INT32_MAX))
        return fail(BSA_ERR_INVALID_ARGUMENT, "nnz=%lld must be in [nqb=%lld, 2^31)", (long long)nnz, (long long)nqb);
    if (!static_ws) {
        const size_t need = bsa_decode_workspace_bytes(batch, heads_q, d);
        if (workspace_bytes < need) return fail(BSA_ERR_CAPACITY, "workspace_bytes %zu < %zu", workspace_bytes, need);
    }

    bsa::DecodeParams p;
    p.q = q; p.k = k_cache; p.v = v_cache; p.o = o; p.lse = lse;
    p.seq_lens = seq_lens; p.row_ptr = spec ? nullptr : row_ptr; p.col_idx = spec ? nullptr : col_idx;
    p.ws = workspace;
    p.rkind = spec ? spec->kind : -1;
    p.n_local = spec ? spec->n_local : 0;
    p.keep_first = spec ? (spec->keep_first != 0) : 0;
    p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.block = block;
    p.n_max = n_max; p.nnz = spec ? 0 : nnz;
    const int G = heads_q / heads_kv;
    p.gc = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
    p.hchunks = G / p.gc;
    // Splits: enough single-wavefront units to cover the device (~1024), but no more than the
    // 32-key sub-blocks of a typical row: the average row of a CSR route (the rows of these
    // routes are of similar length), the row of a full cache for a closed-form one.
    const int64_t base_units = (int64_t)batch * heads_kv * p.hchunks;
    const int64_t row_blocks = spec ? bsa::route_row_count(spec->kind, nqb - 1, spec->n_local, p.keep_first, 0)
                                    : (nnz + nqb - 1) / nqb;
    const int64_t avg_sub = row_blocks * (block / 32);
    int64_t S = (1024 + base_units - 1) / base_units;
    S = S < avg_sub ? S : avg_sub;
    S = S < 1 ? 1 : (S > bsa::kDecodeMaxSplits ? bsa::kDecodeMaxSplits : S);
    p.splits = (int32_t)S;
    if (base_units * S > INT32_MAX || (int64_t)batch * heads_q > INT32_MAX)
        return fail(BSA_ERR_UNSUPPORTED, "grid too large");
    if (static_ws) {
        // the partials of this call: every slot the merge reads is written by the same call, so
        // nothing in the array needs clearing
        const size_t need = (size_t)batch * heads_q * S * (d + 2) * sizeof(float);
        if (need > BSA_STATIC_SCRATCH_BYTES)
            return fail(BSA_ERR_CAPACITY,
                        "decode partials need %zu bytes (batch %d x heads_q %d x %lld splits x (d + 2) floats), "
                        "more than the %zu-byte static scratch array: use bsa_decode_routed with a workspace",
                        need, batch, heads_q, (long long)S, (size_t)BSA_STATIC_SCRATCH_BYTES);
        void* ptr = nullptr;
        const hipError_t e = bsa::static_scratch(&ptr);
        if (e != hipSuccess) return device_error(e, "static scratch lookup");
        p.ws = (float*)ptr;
    }
    const double sc = (scale > 0.f) ? (double)scale : 1.0 / std::sqrt((double)d);
    p.scale_log2 = (float)(sc * 1.4426950408889634073599);
    const hipError_t e = bsa::launch_decode(p, d, dtype == BSA_BF16, stream);
    if (e != hipSuccess) return device_error(e, "decode launch");
    return ok();
}

}  // namespace

bsa_status bsa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int32_t* seq_lens, int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n_max,
                      int32_t d, int32_t block, bsa_dtype dtype, float scale, const int32_t* row_ptr,
                      const int32_t* col_idx, int64_t nnz, float* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    return decode_impl(q, k_cache, v_cache, o, lse, seq_lens, batch, heads_q, heads_kv, n_max, d, block, dtype,
                       scale, row_ptr, col_idx, nnz, nullptr, workspace, workspace_bytes, stream);
}

bsa_status bsa_decode_routed(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                             const int32_t* seq_lens, int32_t batch, int32_t heads_q, int32_t heads_kv,
                             int64_t n_max, int32_t d, int32_t block, bsa_dtype dtype, float scale,
                             const bsa_route_spec* spec, float* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if (!spec) return fail(BSA_ERR_INVALID_ARGUMENT, "spec must be non-NULL");
    return decode_impl(q, k_cache, v_cache, o, lse, seq_lens, batch, heads_q, heads_kv, n_max, d, block, dtype,
                       scale, nullptr, nullptr, 0, spec, workspace, workspace_bytes, stream);
}

bsa_status bsa_decode_routed_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                     const int32_t* seq_lens, int32_t batch, int32_t heads_q, int32_t heads_kv,
                                     int64_t n_max, int32_t d, int32_t block, bsa_dtype dtype, float scale,
                                     const bsa_route_spec* spec, hipStream_t stream) {
    if (!spec) return fail(BSA_ERR_INVALID_ARGUMENT, "spec must be non-NULL");
    return decode_impl(q, k_cache, v_cache, o, lse, seq_lens, batch, heads_q, heads_kv, n_max, d, block, dtype,
                       scale, nullptr, nullptr, 0, spec, nullptr, 0, stream, true);
}

size_t bsa_dense_route_workspace_bytes(int64_t n, int32_t block) {
    if (n < 0 || block < 1) return 0;
    const int64_t nqb = (n + block - 1) / block;
    if (nqb > 65535) return 0;
    return (size_t)(nqb + 1 + nqb * (nqb + 1) / 2) * sizeof(int32_t);
}

size_t bsa_bsbr_workspace_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d,
                                int32_t chunk) {
    if (batch < 0 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv || n < 1 || d < 1 || chunk < 1) return 0;
    const size_t nch = (size_t)((n + chunk - 1) / chunk);
    return align256((size_t)batch * heads_kv * nch * d * d * sizeof(float)) +
           (size_t)batch * heads_q * nch * d * d * sizeof(float);
}

bsa_status bsa_bsbr_forward(const void* q, const void* k, const void* v, const void* r_meta, const void* h_meta,
                            void* o, int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d,
                            int32_t chunk, bsa_dtype dtype, float scale, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    if (batch < 0 || heads_q < 1 || heads_kv < 1 || n < 0 || d < 1 || chunk < 1)
        return fail(BSA_ERR_INVALID_ARGUMENT,
                    "sizes must satisfy batch >= 0, heads >= 1, n >= 0, d >= 1, chunk >= 1 "
                    "(got batch=%d heads_q=%d heads_kv=%d n=%lld d=%d chunk=%d)",
                    batch, heads_q, heads_kv, (long long)n, d, chunk);
    if (heads_q % heads_kv != 0)
        return fail(BSA_ERR_INVALID_ARGUMENT, "heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
    if (dtype != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "BSBR supports bf16 only");
    if (d != 64 && d != 128) return fail(BSA_ERR_UNSUPPORTED, "head dim d=%d not supported (64 or 128)", d);
    if (chunk != 64 && chunk != 128) return fail(BSA_ERR_UNSUPPORTED, "chunk=%d not supported (64 or 128)", chunk);
    if (!(scale <= 0.f) && !std::isfinite(scale)) return fail(BSA_ERR_INVALID_ARGUMENT, "scale must be finite");
    const int64_t nch = (n + chunk - 1) / chunk;
    if (nch > 1024) return fail(BSA_ERR_UNSUPPORTED, "%lld chunks exceed 1024", (long long)nch);
    if (batch == 0 || n == 0) return ok();
    if (!q || !k || !v || !r_meta || !h_meta || !o || !workspace)
        return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v, r_meta, h_meta, o and workspace must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(r_meta) || !aligned16(h_meta) || !aligned16(o) ||
        !aligned16(workspace))
        return fail(BSA_ERR_INVALID_ARGUMENT, "all tensors and the workspace must be 16-byte aligned");
    const size_t need = bsa_bsbr_workspace_bytes(batch, heads_q, heads_kv, n, d, chunk);
    if (workspace_bytes < need) return fail(BSA_ERR_CAPACITY, "workspace_bytes %zu < %zu", workspace_bytes, need);
    if ((int64_t)batch * heads_q * nch > INT32_MAX || (int64_t)batch * heads_q * nch * d * d / 1024 > INT32_MAX)
        return fail(BSA_ERR_UNSUPPORTED, "grid too large");
    char* ws = (char*)workspace;
    bsa::BsbrParams p;
    p.q = q; p.k = k; p.v = v; p.r = r_meta; p.h = h_meta; p.o = o;
    p.F = (float*)ws;
    ws += align256((size_t)batch * heads_kv * nch * d * d * sizeof(float));
    p.A = (float*)ws;
    p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.nch = (int32_t)nch; p.n = n;
    const double sc = (scale > 0.f) ? (double)scale : 1.0 / std::sqrt((double)d);
    p.scale_log2 = (float)(sc * 1.4426950408889634073599);
    const hipError_t e = bsa::launch_bsbr(p, d, chunk, stream);
    if (e != hipSuccess) return device_error(e, "BSBR launch");
    return ok();
}

bsa_status bsa_dense_causal_ref(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d,
                                int32_t block, bsa_dtype dtype, float scale, int32_t* route_workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    bsa_status s = validate_forward(q, k, v, o, lse, batch, heads_q, heads_kv, n, d, block, dtype, nullptr,
                                    nullptr, 0, false);
    if (s != BSA_OK || batch == 0 || n == 0) return s;
    if (!(scale <= 0.f) && !std::isfinite(scale))
        return fail(BSA_ERR_INVALID_ARGUMENT, "scale must be finite");
    const int64_t nqb = (n + block - 1) / block;
    if (nqb > 65535) return fail(BSA_ERR_UNSUPPORTED, "dense route with %lld blocks exceeds 2^31 entries", (long long)nqb);
    const size_t need = bsa_dense_route_workspace_bytes(n, block);
    if (!route_workspace) return fail(BSA_ERR_INVALID_ARGUMENT, "route_workspace must be non-NULL");
    if (((uintptr_t)route_workspace & 3u) != 0) return fail(BSA_ERR_INVALID_ARGUMENT, "route_workspace must be 4-byte aligned");
    if (workspace_bytes < need)
        return fail(BSA_ERR_CAPACITY, "workspace_bytes %zu < %zu", workspace_bytes, need);
    bsa_route_spec spec;
    memset(&spec, 0, sizeof(spec));
    spec.kind = BSA_ROUTE_DENSE_CAUSAL;
    int32_t* rp = route_workspace;
    int32_t* ci = route_workspace + nqb + 1;
    const hipError_t e = bsa::launch_route_build(spec, nqb, rp, ci, stream);
    if (e != hipSuccess) return device_error(e, "dense route build launch");
    const int64_t nnz = nqb * (nqb + 1) / 2;
    return run_forward(q, k, v, o, lse, batch, heads_q, heads_kv, n, d, block, dtype, scale, rp, ci, nnz, stream);
}

}  // extern "C"
