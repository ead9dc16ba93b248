/*
 * bsa.h — causal block-sparse attention forward (prefill) on AMD Instinct MI355X (gfx950).
 *
 * The operation.  A sequence of n tokens is cut into blocks of B tokens; block b holds
 * tokens [b*B, min((b+1)*B, n)), and there are nqb = ceil(n/B) blocks ("Block Sparse
 * Attention in LLMs", section 3 "Why block sparse?").  A route gives each query block i
 * the list of key blocks it reads — the block mask M_B of "Block-Sparse Attention"
 * ("Math Or Compute Schema"), kept as adjacency lists like the allowed_blocks dictionary
 * of "Block Sparse Attention in LLMs" (section 6 "GPU implementation view").  Per head,
 * the output is exact softmax attention restricted to the route, with the mask applied
 * before the softmax so excluded pairs carry weight exactly zero:
 *
 *     O[t] = sum_s P[t,s] V[s],   P[t,.] = softmax_s( scale * Q[t].K[s]  over s in sel(t) )
 *     sel(t) = { s : s <= t, s < n, floor(s/B) in R(floor(t/B)) }
 *
 * (per-head formula softmax(Q_i K_i^T / sqrt(d_k)) V_i of "Block-Sparse Attention",
 * section "Math Or Compute Schema"; a query block reads itself causally: "BF1: A Causal
 * Dyadic Sparse-Attention Retrofit ...", Method; "bsbr", Solution, mask M_in).
 *
 * Conventions shared by every call:
 *  - All tensor and route pointers are DEVICE pointers owned by the caller (for example
 *    allocated by PyTorch).  The library allocates and frees nothing and keeps no state
 *    apart from a thread-local error string.
 *  - All device work is enqueued asynchronously on the caller's `stream` (NULL = the
 *    default stream); no call synchronises the device unless stated.
 *  - Every call returns a bsa_status and never aborts, exits or throws.  Arguments are
 *    validated on the host before any HIP call, so an invalid call does no device work.
 *    A launch failure reported by the HIP runtime maps to BSA_ERR_DEVICE.
 *    bsa_last_error() returns a human-readable detail for the last non-OK return on the
 *    calling thread.
 *  - Calls are re-entrant; concurrent calls on different streams are independent.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsa_status {
    BSA_OK = 0,
    BSA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, negative size, heads_q % heads_kv != 0 */
    BSA_ERR_UNSUPPORTED = 2,      /* valid but not implemented: head dim, block width or dtype */
    BSA_ERR_BAD_ROUTE = 3,        /* route contents violate the CSR rules (bsa_check_route) */
    BSA_ERR_CAPACITY = 4,         /* a caller buffer is too small */
    BSA_ERR_DEVICE = 5            /* the HIP runtime reported an error */
} bsa_status;

typedef enum bsa_dtype {
    BSA_BF16 = 0, /* bfloat16 inputs and output; fp32 accumulation; bf16 MFMA */
    BSA_FP32 = 1  /* float32 inputs and output; fp32 arithmetic throughout */
} bsa_dtype;

typedef enum bsa_route_kind {
    /* BF1 causal dyadic route ("BF1 ...", Method and section 3.1 "Causal dyadic block graph"):
     * R(i) = {i} u {i-l : 1<=l<=n_local, i-l>=0} u {i-2^k : k>=0, 2^k<=i} u ({0} if keep_first). */
    BSA_ROUTE_BF1 = 0,
    /* BSBR within-chunk term ("bsbr", Solution, mask M_in): R(i) = {i}. */
    BSA_ROUTE_BLOCK_DIAGONAL = 1,
    /* Dense causal attention as a route: R(i) = {0, ..., i}. */
    BSA_ROUTE_DENSE_CAUSAL = 2,
    /* Static-random nonlocal graph (BF1's topology control, "BF1 ...", section 5 "Topology
     * control"; seed 17 in section 8): R(0) = {0}; for i >= 1, R(i) = {i} u ({0} if keep_first)
     * u T(i), where T(i) holds the m = min(n_random, #candidates) candidates j (1..i-1 when
     * keep_first, else 0..i-1) with the smallest (h(seed,i,j), j), h(seed,i,j) =
     * SM(seed ^ SM((i<<32)|j)), SM = first SplitMix64 output from a given state (Steele, Lea &
     * Flood, OOPSLA 2014), all arithmetic on unsigned 64-bit words. */
    BSA_ROUTE_STATIC_RANDOM = 3,
    /* Local sliding band, BF1's equal-budget local control ("BF1 ...", Abstract; section 5
     * "Topology control" and "Communication depth": matched sliding): the block and its
     * n_local predecessors, R(i) = {j : max(0, i - n_local) <= j <= i}.  The fixed band of
     * sliding-window attention, aligned to blocks ("Block-Sparse Attention", comparison with
     * local and sliding-window attention).  n_local = 0 is the block-diagonal route and
     * n_local >= nqb - 1 the dense causal route. */
    BSA_ROUTE_SLIDING_WINDOW = 4
} bsa_route_kind;

/* Route parameters.  Fields a kind does not use are ignored. */
typedef struct bsa_route_spec {
    int32_t kind;       /* bsa_route_kind */
    int32_t n_local;    /* BF1: local predecessors (the BF1 summary uses 2); sliding: band
                           predecessors (the window is n_local + 1 blocks); >= 0 */
    int32_t keep_first; /* BF1, static-random: nonzero keeps block 0 in every row */
    int32_t n_random;   /* static-random: drawn earlier blocks per row (14); >= 0 */
    uint64_t seed;      /* static-random: graph seed (17) */
} bsa_route_spec;

/*
 * bsa_build_route — write the CSR route for n tokens at block width `block`.
 *
 * Output (device, caller-owned):
 *   row_ptr  int32[nqb+1]: row_ptr[0] = 0, row_ptr[i+1] - row_ptr[i] = |R(i)|.
 *   col_idx  int32[nnz]:   row i's key blocks, strictly ascending, so the self block i is last.
 * nnz is computed on the host (closed-form row counts) and written to *nnz_out (host pointer,
 * required).  Size query: when row_ptr == NULL only *nnz_out is written and no device work is
 * done.  Otherwise col_capacity (entries available at col_idx) must be >= nnz, else
 * BSA_ERR_CAPACITY with *nnz_out still set; col_idx may be NULL only when nnz == 0.
 * Requires n >= 0, block >= 1, nqb and nnz < 2^31.  n == 0 writes row_ptr[0] = 0 only.
 * The fill runs as integer kernels on `stream` ("BF1 ...", section 4: topology/planning is
 * timed apart from the attention kernel).
 */
bsa_status bsa_build_route(const bsa_route_spec* spec, int64_t n, int32_t block,
                           int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                           int64_t* nnz_out, hipStream_t stream);

/*
 * bsa_build_route_transpose — the transposed route: row j lists, ascending, the query blocks i
 * whose row of (row_ptr, col_idx) holds key block j (the readers of block j; for a valid route
 * the first entry is j itself).  The gradients of K and V walk these rows (bsa_backward).
 * Input: a route accepted by bsa_check_route, nqb + 1 row pointers, nnz entries (device).
 * Output (device, caller-owned): t_row_ptr int32[nqb+1], t_col_idx int32[nnz] (a valid route
 * transposes to exactly nnz entries).  Integer kernels on `stream`.  Memory-safe on any input:
 * row pointers are read clamped to [0, nnz], every t_row_ptr value is clamped to nnz and no
 * write goes past t_col_idx[nnz - 1], so a malformed route (say, overlapping rows) yields a
 * meaningless but in-bounds transpose; results are defined only for valid routes.
 */
bsa_status bsa_build_route_transpose(const int32_t* row_ptr, const int32_t* col_idx, int64_t nqb, int64_t nnz,
                                     int32_t* t_row_ptr, int32_t* t_col_idx, hipStream_t stream);

/*
 * bsa_forward — block-sparse attention forward over a CSR route (see the top of this file).
 *
 * Layout (device, caller-owned, contiguous, d innermost, 16-byte aligned base pointers):
 *   q, o  [batch, heads_q,  n, d]   in `dtype`
 *   k, v  [batch, heads_kv, n, d]   in `dtype`
 *   lse   float32 [batch, heads_q, n] or NULL: natural-log log-sum-exp of the scaled,
 *         selected scores of each query row.
 * Grouped-query attention: query head h reads key/value head h / (heads_q / heads_kv).
 * scale <= 0 selects 1/sqrt(d).
 * Route (device): row_ptr int32[nqb+1], col_idx int32[nnz] with nqb = ceil(n/block), shared by
 * every batch entry and head.  Rows are read as given; row pointers are clamped to [0, nnz] and
 * entries outside [0, i] are read as block i, so a malformed route cannot make the kernel read
 * out of bounds, but only routes accepted by bsa_check_route give defined results (the bf16
 * kernels take the last entry of a row as its diagonal block).  With the
 * environment variable BSA_VALIDATE_ROUTE=1 the route is copied to the host and checked first
 * (this synchronises `stream`).
 * Supported: d in {64, 128}; block in {64, 128}; dtype BF16 or FP32; any n >= 0 (the last block
 * may be partial; batch == 0 or n == 0 is a no-op).  BF16 output is rounded to nearest-even
 * from fp32; the bf16 path rounds the softmax weights to bf16 before the PV product.
 * Non-finite inputs: a NaN in a q row makes that output row (and its lse) NaN; a NaN in a key
 * or value row reaches the output rows that select that key; rows of the same diagonal block
 * that precede the key may show it too (they share its matrix product); every other output
 * row is bit-identical to the run without it.
 */
bsa_status bsa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                       int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d,
                       int32_t block, bsa_dtype dtype, float scale,
                       const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                       hipStream_t stream);

/*
 * bsa_dense_causal_ref — the same forward kernel over the dense causal route (row i reads
 * 0..i): the dense baseline the BF1 summary measures its speedups against ("BF1 ...",
 * Abstract; section 5 "Per-layer prefill scaling").  The route is built into the caller's
 * device workspace, which must hold bsa_dense_route_workspace_bytes(n, block) bytes
 * (int32[nqb+1] row_ptr followed by int32[nqb(nqb+1)/2] col_idx), else BSA_ERR_CAPACITY.
 * Other arguments as for bsa_forward.
 */
bsa_status bsa_dense_causal_ref(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n,
                                int32_t d, int32_t block, bsa_dtype dtype, float scale,
                                int32_t* route_workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Workspace bytes bsa_dense_causal_ref needs for n tokens at width block (0 on bad input). */
size_t bsa_dense_route_workspace_bytes(int64_t n, int32_t block);

/*
 * bsa_backward — gradients of bsa_forward (the "gradients" correctness gate of "BF1 ...",
 * section 4).  With P the forward's weights (recomputed from q, k and its log-sum-exp) and
 * D[t] = sum_d d_o[t, d] o[t, d]:
 *
 *     dv = P^T d_o,   dS = P * (d_o v^T - D),   dq = scale * dS k,   dk = scale * dS^T q
 *
 * per head, dk and dv summed over the query heads sharing a key/value head (h / G).  Excluded
 * pairs carry no gradient.
 * Inputs (device, caller-owned, contiguous, 16-byte aligned): q, k, v, o, d_o as for
 * bsa_forward (o its output, d_o the upstream gradient of o, same shape); lse float32
 * [batch, heads_q, n] from bsa_forward (required); the route (row_ptr, col_idx, nnz) and its
 * transpose from bsa_build_route_transpose (t_row_ptr, t_col_idx).  Outputs: dq like q, dk and
 * dv like k and v, in `dtype`.  workspace: float32 scratch of at least
 * bsa_backward_workspace_bytes(...) bytes (D and lse scaled to base 2 over rows padded to whole
 * blocks, the segment table of the transposed rows, and fp32
 * partial dk/dv of key blocks whose readers are split over several work-groups); its contents
 * on entry do not matter.  Supported: dtype BF16; d in {64, 128}; block in {64, 128}; any n >= 0.
 * Four kernels on `stream`; the result is deterministic (no atomics).
 */
bsa_status bsa_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                        const float* lse, void* dq, void* dk, void* dv, int32_t batch, int32_t heads_q,
                        int32_t heads_kv, int64_t n, int32_t d, int32_t block, bsa_dtype dtype, float scale,
                        const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                        const int32_t* t_row_ptr, const int32_t* t_col_idx,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes bsa_backward needs (0 on bad input). */
size_t bsa_backward_workspace_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d,
                                    int32_t block, int64_t nnz);

/*
 * bsa_decode — selected-page decode: one new query token per sequence against the key/value
 * blocks of its route row ("BF1 ...", section 5 "Selected-page decode characterization"; the
 * "decode-reference agreement" gate of section 4).  Sequence b holds seq_lens[b] tokens in its
 * cache; its newest token t = seq_lens[b] - 1 (query block i = t / block) attends to the keys
 * s <= t with floor(s / block) in R(i):
 *
 *     o[b, h] = sum_s P[s] v_cache[b, h/G, s],  P = softmax_s( scale * q[b, h] . k_cache[b, h/G, s] )
 *
 * which is row t of bsa_forward's output for that token (G = heads_q / heads_kv).
 *
 * Layout (device, caller-owned, contiguous, 16-byte aligned):
 *   q, o              [batch, heads_q, d]          in `dtype`
 *   k_cache, v_cache  [batch, heads_kv, n_max, d]  in `dtype` (rows >= seq_lens[b] are not read)
 *   lse               float32 [batch, heads_q] or NULL (natural log)
 *   seq_lens          int32 [batch] on the device; values are clamped to [1, n_max]
 *   row_ptr, col_idx  the CSR route for n_max tokens at width `block` (as for bsa_forward):
 *                     built once for the cache capacity, it serves every length up to n_max
 *   workspace         float32 partials, at least bsa_decode_workspace_bytes(batch, heads_q, d)
 *                     bytes, else BSA_ERR_CAPACITY; its contents on entry do not matter
 * scale <= 0 selects 1/sqrt(d).  Supported: d in {64, 128}; block in {64, 128}; dtype BF16 or
 * FP32; n_max >= 1; batch == 0 is a no-op.  fp32 arithmetic throughout (the softmax weights are
 * not rounded); the output is rounded once to `dtype`.  Two kernels on `stream`.
 */
bsa_status bsa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int32_t* seq_lens, int32_t batch, int32_t heads_q, int32_t heads_kv,
                      int64_t n_max, int32_t d, int32_t block, bsa_dtype dtype, float scale,
                      const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                      float* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes bsa_decode needs (0 on bad input). */
size_t bsa_decode_workspace_bytes(int32_t batch, int32_t heads_q, int32_t d);

/*
 * bsa_decode_routed — bsa_decode with the route given by its parameters instead of a CSR
 * route: each sequence's row R(i) is generated inside the kernel from the closed form of the
 * kind (the sets documented at bsa_route_kind), so a decode step needs no route in memory and
 * no planning launch ("BF1 ...", section 4: topology/planning cost kept apart from the
 * attention kernel; here that cost is zero).  Same arguments, layout, arithmetic and output as
 * bsa_decode, with `spec` (host pointer, read during the call only) in place of row_ptr,
 * col_idx and nnz.  Kinds: BF1, block-diagonal, dense causal, sliding window; static-random
 * returns BSA_ERR_UNSUPPORTED (its rows come from a per-row selection: build the route with
 * bsa_build_route and call bsa_decode), an unknown kind or n_local < 0 BSA_ERR_INVALID_ARGUMENT.
 * The output equals bsa_decode's with the route bsa_build_route writes for the same spec,
 * bit for bit when both calls choose the same number of key splits (the split count follows
 * the average row of a CSR route and the row of a full cache here).  Two kernels on `stream`.
 */
bsa_status bsa_decode_routed(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                             const int32_t* seq_lens, int32_t batch, int32_t heads_q, int32_t heads_kv,
                             int64_t n_max, int32_t d, int32_t block, bsa_dtype dtype, float scale,
                             const bsa_route_spec* spec, float* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * bsa_decode_routed_noalloc — bsa_decode_routed without a workspace argument, for callers that
 * cannot allocate device memory: code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The fp32 partials go to the library's static scratch array instead, a
 * device-resident array of BSA_STATIC_SCRATCH_BYTES that every device the library runs on holds
 * from its first call until the process ends.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine).  Same arguments (minus workspace and
 * workspace_bytes), kernels, arithmetic and output as bsa_decode_routed: bit for bit equal to it.
 * Limit: the partials need batch * heads_q * splits * (d + 2) * 4 bytes, where the split count
 * (at most 64) is the one bsa_decode_routed chooses; beyond BSA_STATIC_SCRATCH_BYTES the call
 * returns BSA_ERR_CAPACITY before any device work (e.g. at d = 128 and 64 splits, up to 252
 * (batch, query head) pairs).  Every slot the merge reads is written by the same call, so the
 * array's contents on entry do not matter.  All calls on one device share its array: calls that
 * overlap in time on one device (on different streams, or from different threads without
 * ordering) race and give undefined results; calls ordered on one stream are safe.
 * Errors: as bsa_decode_routed, plus BSA_ERR_CAPACITY (array too small) and BSA_ERR_DEVICE
 * (symbol lookup or launch failure).
 */
#define BSA_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
bsa_status bsa_decode_routed_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                     const int32_t* seq_lens, int32_t batch, int32_t heads_q, int32_t heads_kv,
                                     int64_t n_max, int32_t d, int32_t block, bsa_dtype dtype, float scale,
                                     const bsa_route_spec* spec, hipStream_t stream);

/*
 * bsa_bsbr_forward — BSBR attention ("bsbr", Solution: the combined formula), chunks of
 * `chunk` tokens, nch = ceil(n / chunk):
 *
 *     O[t] = softmax-attention of t over the earlier tokens of its own chunk (causal)
 *          + Q[t]^T A_c(t),   A_c = sum over c' < c of W[c, c'] F_c',
 *     F_c = K_c^T V_c (d x d, the chunk's tokens),  W[c, :] = softmax over c' < c of
 *     scale * R_c . H_c'  (chunk 0 retrieves nothing).
 *
 * The within-chunk term is the causal block-diagonal attention (bsa_forward with the
 * block-diagonal route computes the same term); both terms are formed by one kernel per chunk.
 * Inputs (device, caller-owned, contiguous, 16-byte aligned, bf16): q [batch, heads_q, n, d];
 * k, v [batch, heads_kv, n, d]; r_meta (meta queries) [batch, heads_q, nch, d]; h_meta (meta
 * keys) [batch, heads_kv, nch, d].  Output o like q.  scale <= 0 selects 1/sqrt(d) for both
 * softmaxes.  workspace: at least bsa_bsbr_workspace_bytes(...) bytes (fp32 chunk states per
 * key/value head and retrieved states per query head); contents on entry do not matter.
 * Supported: BF16; d in {64, 128}; chunk in {64, 128}; 1 <= nch <= 1024.  Three kernels on
 * `stream`, no atomics.
 * Errors: BSA_ERR_INVALID_ARGUMENT (NULL or misaligned pointers, bad sizes), BSA_ERR_UNSUPPORTED
 * (dtype, d, chunk, nch), BSA_ERR_CAPACITY (workspace), BSA_ERR_DEVICE (launch failure).
 */
bsa_status bsa_bsbr_forward(const void* q, const void* k, const void* v, const void* r_meta,
                            const void* h_meta, void* o, int32_t batch, int32_t heads_q,
                            int32_t heads_kv, int64_t n, int32_t d, int32_t chunk, bsa_dtype dtype,
                            float scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes bsa_bsbr_forward needs (0 on bad input). */
size_t bsa_bsbr_workspace_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t n, int32_t d,
                                int32_t chunk);

/*
 * bsa_check_route — validate a CSR route held in HOST memory: row_ptr[0] == 0, row_ptr
 * non-decreasing, row_ptr[nqb] == nnz, and every row strictly ascending within [0, i] and
 * ending with i (the self block is mandatory, so no row is empty).  BSA_OK or
 * BSA_ERR_BAD_ROUTE (detail in bsa_last_error).  Pure host code.
 */
bsa_status bsa_check_route(const int32_t* row_ptr, const int32_t* col_idx, int64_t nqb, int64_t nnz);

/* Static name of a status code. */
const char* bsa_status_string(bsa_status s);

/* Detail for the last non-OK return on the calling thread ("" if none). */
const char* bsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
