/*
 * moe_mi355x.h -- C ABI of the MI355X (gfx950) forward pass of a LongCat-Flash
 * Mixture-of-Experts layer: a pool of N SwiGLU FFN experts plus Z
 * zero-computation (identity) experts, a per-expert selection bias, top-K
 * routing, expert-grouped FFN GEMMs, identity passthrough and a compensated,
 * gate-weighted combine.
 *
 * Source of the method: LongCat-Flash Technical Report notes, "Key claims"
 * and "Method" (report §2.1 zero-computation experts and the PID-adjusted
 * expert bias, §2.2 dispatch/combine, §2.3.2 Eq. 8 variance compensation,
 * §2.4 model configuration: K = 12 of 512 FFN + 256 zero experts, hidden
 * 6144, expert intermediate 2048).
 *
 * Conventions shared by every call
 *   - Every pointer argument is DEVICE memory owned by the caller; the library
 *     never allocates, frees or keeps a pointer after the call returns.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream) and returns without synchronising.
 *     The calling thread's current HIP device must be the one the pointers
 *     and the stream belong to.
 *     Calls on one stream may follow each other with no host round trip:
 *     data-dependent sizes (rows per expert) stay on the device.
 *   - Arguments are validated on the host BEFORE any HIP call; a failed check
 *     returns a status and enqueues nothing.  A launch failure returns
 *     MOE_ERR_LAUNCH.  No call aborts the process.
 *   - Layouts are row-major.  Expert ids: FFN experts 0..n_ffn-1, identity
 *     experts n_ffn..E-1.  Routing tensors (logits, bias, gates, y_acc) are
 *     fp32, index tensors int32.  Activations, expert weights and the layer
 *     output share one dtype: MOE_F32 or MOE_BF16 (fp32 accumulation always).
 *   - Pointers to bf16 data must be 16-byte aligned, other pointers 4-byte
 *     aligned (MOE_ERR_ALIGN).  T*K must stay below 2^31.
 *   - Results are bitwise deterministic run to run (no floating-point
 *     atomics), the property the report's SDC detection relies on (report §1,
 *     §3.1.3).
 *   - Calls that share a workspace must be ordered on one stream.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,      /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,     /* a size is out of range or not a supported multiple */
    MOE_ERR_DTYPE = 3,     /* unknown dtype */
    MOE_ERR_ALIGN = 4,     /* a pointer is not aligned as required */
    MOE_ERR_WORKSPACE = 5, /* workspace smaller than the *_workspace_bytes query */
    MOE_ERR_LAUNCH = 6,    /* a HIP launch failed (hipGetLastError) */
    MOE_ERR_TOO_LARGE = 7  /* the sizes need more than a fixed scratch holds */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Router scores of every expert of the pool (Technical Report notes, Key
 * claims [§2.1, §2.4]: the router picks from one pool of FFN + zero experts).
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h], fp32 result.
 * x: [T][H] in x_dtype; w_router: [E][H] fp32; logits: [T][E] fp32.
 * Any T, E, H >= 1; x and w_router element-aligned.  With bf16 x, H % 64 ==
 * 0 and x and w_router 16-byte aligned, the scores run on bf16 matrix cores
 * with w_router split exactly into three bf16 planes (every product exact,
 * fp32 accumulation); otherwise on fp32 FMA. */
moe_status moe_router_logits(const void *x, int x_dtype, const float *w_router,
                             int T, int H, int E, float *logits, void *stream);

/* The router weights' three bf16 planes, split once (the same exact split
 * moe_router_logits does on every call: w = hi + mid + lo, hi = w truncated
 * to bf16, mid = the remainder truncated, lo = what is left; Technical Report
 * notes, Key claims [§2.1]: fp32 router scores).  A weight-format
 * preparation, to be redone whenever w_router changes.
 *   w_router [E][H] fp32 (16-byte aligned), w_planes [3][E][H] bf16 (16-byte
 *   aligned, caller-owned: plane p of expert e at (p*E + e)*H).
 * H % 8 == 0, E >= 1. */
moe_status moe_router_split_weights(const float *w_router, int E, int H, void *w_planes,
                                    void *stream);

/* moe_router_logits with the planes of moe_router_split_weights: bitwise the
 * same logits (the same matrix-core operations in the same order), without
 * the split in the kernel where the large-batch tiles run (bf16 x, H % 32 ==
 * 0, at least 256 tiles of 256 tokens x 96 experts).  w_router is still
 * required (the other tile shapes split it themselves); w_planes may be
 * NULL, which is moe_router_logits.  w_planes stale against w_router gives
 * scores of the weights it was split from. */
moe_status moe_router_logits_planes(const void *x, int x_dtype, const float *w_router,
                                    const void *w_planes, int T, int H, int E, float *logits,
                                    void *stream);

/* Top-K routing with a selection bias (Technical Report notes, Key claims
 * [§2.1.1]: the bias the PID controller adjusts from routing frequency enters
 * selection only).
 *   key[t][e] = logits[t][e] + bias[e]         (one fp32 addition)
 *   topk_idx[t][k]: the K largest keys, in descending key order; equal keys go
 *     to the lower expert id (-0.0 equals +0.0; -inf is a valid key, i.e. a
 *     masked expert; a NaN key ranks below -inf).
 *   topk_gate[t][k] = softmax over all E unbiased logits, taken at the chosen
 *     expert; not renormalised over the K picks.
 *   counts[e] = number of tokens that chose e (the routing-frequency
 *     histogram), overwritten (not accumulated).
 *   dev_status (may be NULL): an int32 the kernels set to 1 when a token's
 *     choice or gates are undefined: a NaN key, a +inf or NaN logit, or every
 *     logit of the token -inf (a -inf logit or key alone is a masked expert,
 *     not an error); they never clear it -- the caller zeroes it.
 * logits [T][E], bias [E], topk_idx/topk_gate [T][K], counts [E].
 * 1 <= K <= E <= 1024, T >= 1. */
moe_status moe_route(const float *logits, const float *bias, int T, int E, int K,
                     int32_t *topk_idx, float *topk_gate, int32_t *counts,
                     int32_t *dev_status, void *stream);

/* Dispatch on one GPU: group every FFN selection by expert (Technical Report
 * notes, Key claims [§2.2], the dispatch half of dispatch/combine).
 * Rows are expert-major and, within an expert, in ascending token order.
 *   offsets[e] = first row of expert e, offsets[n_ffn] = S (FFN rows)
 *   x_perm[r] = x[t] for the selection (t, k) held by row r, r < S
 *   row_src[r] = t*K + k, r < S
 *   slot_row[t*K + k] = its row, or -1 when it chose an identity expert
 * x: [T][H] (dtype); topk_idx: [T][K] with entries in [0, E) (an id outside
 * [0, n_ffn) is an identity pick: slot_row -1, no row); counts: the
 * histogram moe_route wrote for these topk_idx (entries 0..n_ffn-1 are
 * read); x_perm: capacity [T*K][H]; row_src: capacity [T*K]; slot_row:
 * [T*K]; offsets: [n_ffn + 1].
 * Rows >= S of x_perm and row_src are left untouched.
 * x_perm may be NULL (and then x too): only offsets, row_src and slot_row are
 * written, for moe_expert_ffn_gather, which reads the rows from x itself.
 * counts that are not the histogram of topk_idx give a meaningless grouping
 * but no access outside the buffers (every row is clamped into [0, T*K)).
 * No workspace: each 64-token block counts the picks it needs itself. */
moe_status moe_permute(const void *x, int dtype, const int32_t *topk_idx, const int32_t *counts,
                       int T, int H, int K, int n_ffn, int32_t *offsets, void *x_perm,
                       int32_t *row_src, int32_t *slot_row, void *stream);

/* The FFN experts on their grouped rows (Technical Report notes, Key claims
 * [§2.4]: fine-grained FFN experts of intermediate size I; SwiGLU form).
 * For every expert e with rows [offsets[e], offsets[e+1]) (empty experts cost
 * nothing):
 *   hh = silu(X W_g^T) * (X W_u^T),  silu(a) = a / (1 + exp(-a))
 *   y_perm rows = hh W_d^T
 * w13: [n_ffn][2I][H] (rows 0..I-1 = W_g, I..2I-1 = W_u); w2: [n_ffn][H][I];
 * x_perm, y_perm: [rows_cap][H]; offsets as written by moe_permute, with
 * offsets[n_ffn] <= rows_cap.  Only rows < offsets[n_ffn] of y_perm are
 * written.  fp32 accumulation; for MOE_BF16, hh is rounded to bf16 between
 * the two GEMMs and y_perm is stored in bf16.
 * MOE_BF16 requires H % 128 == 0 and I % 64 == 0.
 * n_ffn == 0 (a pool of zero-computation experts only) enqueues nothing;
 * w13 and w2 may then be NULL.
 * ws: at least moe_expert_ffn_workspace_bytes(rows_cap, n_ffn, I, dtype). */
size_t moe_expert_ffn_workspace_bytes(int rows_cap, int n_ffn, int I, int dtype);
moe_status moe_expert_ffn(const void *x_perm, const int32_t *offsets, int rows_cap,
                          int n_ffn, int H, int I, const void *w13, const void *w2,
                          int dtype, void *y_perm, void *ws, size_t ws_bytes,
                          void *stream);

/* moe_expert_ffn with the dispatch copy folded into the first GEMM's loads
 * (the same Key claims [§2.2] dispatch and [§2.4] experts): row r's
 * activations are read straight from token row row_src[r] / K of x, so
 * x_perm never needs to exist and moe_permute may be called with
 * x_perm = NULL.  y_perm and the results are those of moe_expert_ffn on the
 * x_perm moe_permute would have written, bit for bit.
 * x: [T][H] (dtype, 16-byte aligned for MOE_BF16); row_src: capacity
 * [rows_cap], as written by moe_permute, entries in [0, T*K) (others are
 * clamped to a token row in [0, T), never read out of bounds); the other
 * arguments, limits and errors as for moe_expert_ffn, plus MOE_ERR_SHAPE for
 * T < 1, K < 1 or T*K >= 2^31. */
moe_status moe_expert_ffn_gather(const void *x, int T, int K, const int32_t *row_src,
                                 const int32_t *offsets, int rows_cap, int n_ffn, int H,
                                 int I, const void *w13, const void *w2, int dtype,
                                 void *y_perm, void *ws, size_t ws_bytes, void *stream);

/* moe_expert_ffn_gather for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels, with the workspace (the m-tile list and the
 * bf16 hh rows between the two GEMMs) taken from a fixed scratch array that
 * the library holds on every GPU it runs on until the process ends, instead
 * of a caller-allocated ws.  Nothing is allocated by the call.
 *   Limit: moe_expert_ffn_workspace_bytes(rows_cap, n_ffn, I, dtype) must
 *   not exceed MOE_EXPERT_FFN_NOALLOC_SCRATCH_BYTES (32 MiB: e.g. rows_cap
 *   up to ~8,000 FFN rows at I = 2048, i.e. decode-sized batches), else
 *   MOE_ERR_TOO_LARGE and nothing is enqueued.
 *   Every call on one GPU uses that GPU's one scratch array: calls that
 *   overlap on one GPU (other streams, other threads) race and must be
 *   ordered, e.g. on one stream.  The scratch needs no clearing: each call
 *   writes the parts it reads.  The first call on a device looks up the
 *   array's address there (a runtime query, not an allocation).
 * Arguments, results (bit for bit those of moe_expert_ffn_gather) and the
 * other errors as for moe_expert_ffn_gather, without ws and ws_bytes. */
#define MOE_EXPERT_FFN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
moe_status moe_expert_ffn_gather_noalloc(const void *x, int T, int K, const int32_t *row_src,
                                         const int32_t *offsets, int rows_cap, int n_ffn, int H,
                                         int I, const void *w13, const void *w2, int dtype,
                                         void *y_perm, void *stream);

/* Zero-computation experts (Technical Report notes, Key claims [§2.1]:
 * identity experts return their input):
 *   y_acc[t][h] = (sum over slots k with topk_idx >= n_ffn of topk_gate[t][k]) * x[t][h]
 * x: [T][H] (dtype); topk_idx, topk_gate: [T][K]; y_acc: [T][H] fp32. */
moe_status moe_zero_experts(const void *x, int dtype, const int32_t *topk_idx,
                            const float *topk_gate, int T, int H, int K, int n_ffn,
                            float *y_acc, void *stream);

/* Combine (Technical Report notes, Key claims [§2.2] the combine half;
 * [§2.3.2 Eq. 8] the variance-compensation factor on FFN expert outputs):
 *   y[t] = y_acc[t] + sum over slots k with slot_row >= 0, in slot order, of
 *          (ffn_scale * topk_gate[t][k]) * y_perm[slot_row[t*K + k]]
 * accumulated in fp32, then stored in dtype (bf16: round to nearest even).
 * y_perm: rows as written by moe_expert_ffn; slot_row as written by
 * moe_permute; y_acc from moe_zero_experts; y: [T][H] (dtype). */
moe_status moe_combine(const void *y_perm, int dtype, const int32_t *slot_row,
                       const float *topk_gate, float ffn_scale, const float *y_acc,
                       int T, int H, int K, void *y, void *stream);

/* moe_zero_experts and moe_combine in one pass (the same Key claims [§2.1]
 * identity experts, [§2.2] combine, [§2.3.2 Eq. 8] compensation):
 *   y[t] = (sum over slots k with slot_row < 0, in slot order, of
 *           topk_gate[t][k]) * x[t]
 *        + sum over slots k with slot_row >= 0, in slot order, of
 *          (ffn_scale * topk_gate[t][k]) * y_perm[slot_row[t*K + k]]
 * in fp32, stored in dtype.  The identity slots are the ones moe_permute
 * marks -1, i.e. the picks of experts >= n_ffn.  The fp32 operations and
 * their order are those of the two calls, so y is bitwise the same; y_acc is
 * neither needed nor written (4H bytes per token less each way).
 * x: [T][H] (dtype); y_perm, slot_row, topk_gate, y, limits and errors as for
 * moe_combine. */
moe_status moe_combine_identity(const void *y_perm, const void *x, int dtype,
                                const int32_t *slot_row, const float *topk_gate,
                                float ffn_scale, int T, int H, int K, void *y,
                                void *stream);

/* The whole layer in one call (Technical Report notes, Key claims [§2.1]
 * router over one pool of FFN and zero-computation experts with the
 * selection bias, [§2.2] dispatch and combine, [§2.3.2] compensation factor
 * on the FFN outputs, [§2.4] shapes): the five calls of the default path,
 * enqueued on `stream` in this order with the intermediate tensors in `ws`:
 *   moe_router_logits_planes (w_planes may be NULL: moe_router_logits),
 *   moe_route, moe_permute (indices only), moe_expert_ffn_gather with
 *   rows_cap = T*K, moe_combine_identity.
 * y is bitwise the y of those five calls.
 *   x [T][H] (dtype), w_router [E][H] fp32, w_planes [3][E][H] bf16 or NULL,
 *   bias [E] fp32, w13 [n_ffn][2I][H] and w2 [n_ffn][H][I] (dtype; may be
 *   NULL when n_ffn == 0), y [T][H] (dtype), dev_status as for moe_route
 *   (may be NULL).  Expert ids 0..n_ffn-1 are FFN experts, n_ffn..E-1
 *   identity experts.
 *   ws: at least moe_forward_workspace_bytes(T, H, E, n_ffn, I, K, dtype)
 *   bytes, 256-byte aligned, caller-owned; it holds, in order and each
 *   256-byte aligned, logits [T][E] fp32, topk_idx and topk_gate [T][K],
 *   counts [E], offsets [n_ffn+1], row_src and slot_row [T*K], y_perm
 *   [T*K][H] (dtype) and the expert GEMMs' workspace, which the caller may
 *   read after the call.
 * Every check of the five calls runs first: MOE_ERR_NULL, MOE_ERR_DTYPE,
 * MOE_ERR_SHAPE (T, H, E, K, n_ffn, I out of the ranges the five calls take:
 * H % 8, 1 <= K <= E <= 1024, n_ffn <= E; bf16: H % 128, I % 64),
 * MOE_ERR_ALIGN (x, y, w_planes 16 bytes; bf16 weights 16 bytes, fp32 ones
 * 4; ws 256), MOE_ERR_WORKSPACE; a failed check enqueues nothing.
 * moe_forward_workspace_bytes returns 0 for sizes out of range. */
size_t moe_forward_workspace_bytes(int T, int H, int E, int n_ffn, int I, int K, int dtype);
moe_status moe_forward(const void *x, int dtype, const float *w_router, const void *w_planes,
                       const float *bias, const void *w13, const void *w2, int T, int H, int E,
                       int n_ffn, int I, int K, float ffn_scale, void *y, int32_t *dev_status,
                       void *ws, size_t ws_bytes, void *stream);

/* Bias controller (Technical Report notes, Key claims [§2.1.1, §2.1.2] and
 * Method: each FFN expert's selection bias is adjusted from token-routing
 * frequency by a PID controller so that the average number of activated FFN
 * experts per token holds a target; zero-computation experts are excluded).
 * One update from a batch's counts (as written by moe_route for T tokens):
 * for i in 0..n_ffn-1,
 *   err_i       = target / n_ffn - counts[i] / T
 *   integral[i] = integral[i] + err_i
 *   bias[i]     = bias[i] + kp * err_i + ki * integral[i] + kd * (err_i - prev_err[i])
 *   prev_err[i] = err_i
 * bias[n_ffn..E-1] (the zero-computation experts) is not read or written.
 * target: FFN experts activated per token (0 < target <= K in practice).
 * counts: [>= n_ffn] int32; bias: [>= n_ffn] fp32 (the array moe_route
 * reads); integral, prev_err: [n_ffn] fp32 controller state, owned by the
 * caller, zero before the first update.  fp32 arithmetic.
 * MOE_ERR_SHAPE: T < 1, n_ffn outside 1..4096, or a non-finite target or gain. */
moe_status moe_bias_update(const int32_t *counts, int T, int n_ffn, float target, float kp,
                           float ki, float kd, float *bias, float *integral, float *prev_err,
                           void *stream);

/* Router weight similarity (Technical Report notes, Key claims and Method
 * [§3.1.3 Router Stability]: the pairwise cosine similarity of the experts'
 * router weight vectors is tracked as a router-stability diagnostic; high
 * values mark a router collapsed by the load-balance term).
 *   sim[i][j] = <w_i, w_j> / (|w_i| * |w_j|)   for rows w_i of w_router,
 *               0 when either row has zero norm (the diagonal too);
 *   *mean     = average of sim[i][j] over the E*(E-1) pairs i != j
 *               (0 when E = 1).
 * w_router: [E][H] fp32, 16-byte aligned, H % 4 == 0 (pass the first n_ffn
 * rows to restrict the diagnostic to the FFN experts).  sim: [E][E] fp32,
 * exactly symmetric.  mean: one fp32 in device memory.  fp32 products and
 * accumulation on the matrix cores, the row sums and the mean in fp64.
 * ws: at least moe_router_similarity_workspace_bytes(E, H) bytes, 256-byte
 * aligned (partial Gram tiles, norms and row sums; contents need not be
 * initialised).
 * MOE_ERR_SHAPE: E or H < 1, H % 4 != 0, or E*E >= 2^31. */
size_t moe_router_similarity_workspace_bytes(int E, int H);
moe_status moe_router_similarity(const float *w_router, int E, int H, float *sim, float *mean,
                                 void *ws, size_t ws_bytes, void *stream);

/* Diagnostics (not part of the layer): opt-in per-kernel timing.  While
 * enabled, each kernel the calls above enqueue is bracketed by two HIP events
 * recorded on its stream.  moe_profile_enable(1) starts a new session (the
 * previous records are dropped), (0) stops recording; it returns the previous
 * state.  moe_profile_summary waits for the recorded events and writes one
 * line "kernel_name launches total_ms" per kernel into buf (at most len
 * bytes, NUL-terminated); it returns the length of the full text, or -1 if an
 * event could not be read.  moe_profile_select restricts the timing to the
 * kernels named in a comma-separated list (NULL or "": every kernel) and
 * returns the number of names; each bracketed launch costs a few
 * microseconds of stream time, so timed loops select what they need.  The
 * session is process-wide; concurrent callers share it.
 * Graph capture: while the timing is off (the default) a launch reads one
 * atomic flag and records nothing, so every call above can be captured into
 * a HIP graph.  Do not enable it around a capture: the events recorded then
 * become graph nodes, the session's records refer to events that only the
 * graph's replays complete, and moe_profile_summary may report -1. */
int moe_profile_enable(int on);
int moe_profile_select(const char *names);
int moe_profile_summary(char *buf, size_t len);

/* Human-readable name of a status code (static storage). */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
