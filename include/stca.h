/*
 * stca.h -- C ABI of libstca: the Stacked Target Cross Attention (STCA) forward pass
 * on AMD Instinct MI355X (CDNA4, gfx950).
 *
 * Method (web pages on the STCA paper, "Make It Long, Keep It Fast: End-to-End
 * 10k-Sequence Modeling at Billion Scale on Douyin", WWW'26, arXiv 2511.06077):
 *   eq. (1)  SwiGLUFFN(x) = ((x W_u) * SiLU(x W_v)) W_o            (W_u, W_v: d x rd, W_o: rd x d;
 *            the three-matrix reading of the review page, section 2.2; no biases)
 *   eq. (2)  X~(i) = LN(SwiGLUFFN(i)(X))                  per history token, every layer from raw X
 *   eq. (3)  q(1)  = LN(SwiGLUFFN(1)(x_t))
 *   eq. (13) u_j = (q W_Q,j) W_K,j^T,  alpha_j = softmax(u_j X~^T / sqrt(d_h)),  o_j = (alpha_j X~) W_V,j
 *            (the reordered form of the single-query cross attention of eqs. (4)-(5), (12))
 *   eq. (6)  o(i) = [o_1 || ... || o_h] W_O
 *   eq. (7)  q(i+1) = SwiGLUFFN(i+1)([o(1) || ... || o(i) || x_t] W_C(i+1)),  W_C(i+1): (i+1)d x d
 *   eq. (8)  Z = [o(1); ...; o(M)]  per target
 * Request level batching (section 2.2 of the same notes): the targets of one user share that
 * user's history, which is encoded once; users are ragged segments described by offset arrays.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns all memory; the library
 *     allocates nothing and is reentrant.  Its only global state is the fixed scratch array of
 *     stca_attend_noalloc (64 MiB per GPU, in the library's code object) and, on the host, that
 *     array's per-device address, looked up once under a lock.  Device pointers must be 16-byte
 *     aligned (STCA_E_ALIGN otherwise).
 *   - Matrices are row-major.  Storage type of X, x_t, X~ and of every weight matrix is
 *     dims->dtype (fp32 or bf16); LayerNorm gamma/beta, q, o and Z are always fp32.  All
 *     arithmetic accumulates in fp32.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream).  Outputs are
 *     valid once the stream has reached the call's end.  No call synchronises the device.
 *   - Every argument error the host can see is returned as a negative stca_status BEFORE any
 *     work is enqueued.  A failed launch returns STCA_E_HIP (stca_last_error() has the detail).
 *   - Offsets are caller contract: hist_off/tgt_off start at 0, are nondecreasing, end at
 *     total_L/total_T, and no user exceeds max_L history rows or max_T targets.  A user with no
 *     targets is allowed; a user with an empty history (softmax over no tokens is undefined) gets
 *     NaN outputs for its targets.  The ragged kernels check the offsets on the device before they
 *     use them: a batch that breaks the contract makes stca_forward / stca_attend write NaN to
 *     every output row (stca_backward: meaningless gradients) rather than touch memory outside
 *     their buffers.  stca_validate_batch reports which condition a batch breaks.
 */
#ifndef STCA_H
#define STCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STCA_MAX_M 8 /* most stacked layers a call accepts (the pages stack up to 4) */

#if defined(__GNUC__)
#define STCA_API __attribute__((visibility("default")))
#else
#define STCA_API
#endif

typedef enum {
  STCA_OK = 0,
  STCA_E_ARG = -1,       /* NULL pointer, negative size, bad layer index, ... */
  STCA_E_DIMS = -2,      /* unsupported d / h / r / M / dtype combination */
  STCA_E_WORKSPACE = -3, /* workspace NULL or smaller than the *_workspace_size result */
  STCA_E_ALIGN = -4,     /* a device pointer is not 16-byte aligned */
  STCA_E_HIP = -5        /* a HIP runtime call or kernel launch failed */
} stca_status;

typedef enum { STCA_F32 = 0, STCA_BF16 = 1 } stca_dtype;

/* Model sizes.  Supported: d in {64, 128, 256, 512}; h divides d; 1 <= r <= 8; 1 <= M <= STCA_MAX_M.
 * dtype STCA_BF16 runs the MFMA path (bf16 storage, bf16 matrix-core products, fp32 accumulation);
 * STCA_F32 runs the fp32 debug path: fp32 storage, products and accumulation throughout, the
 * larger products on the fp32 matrix cores (v_mfma_f32_32x32x2_f32), the rest on the vector ALU. */
typedef struct {
  int32_t d, h, M, r;
  int32_t dtype;      /* stca_dtype */
  float ln_eps;       /* LayerNorm epsilon (biased variance); must be > 0 */
  int32_t query_ln;   /* 1: apply the layer's LayerNorm after the FFN of eq. (7); 0: as printed */
  int32_t attn_chunk; /* history tokens per attention work item, multiple of 32; 0 = automatic */
  int32_t encode_layers; /* bf16 history encodes of stca_forward (eq. (2)): 1 = one launch per layer,
                          * each followed by that layer's attention; 2 = every layer in one launch
                          * that reads each tile of X once (M encoded buffers in the workspace);
                          * 0 = automatic (2 where one layer's X~ exceeds 1 GiB at d <= 256).
                          * Results are identical either way. */
} stca_dims;

/* One SwiGLU FFN + LayerNorm block (eqs. (1)-(3), (7)).  Wu, Wv: d x rd; Wo: rd x d (dtype);
 * gamma, beta: d floats.  gamma/beta may be NULL only where no LayerNorm is applied. */
typedef struct {
  const void *Wu, *Wv, *Wo;
  const float *gamma, *beta;
} stca_ffn;

/* All parameters of an M-layer stack; index i = 0..M-1 is the pages' layer i+1.
 *   hist[i]  : FFN + LN encoding the history for layer i (eq. (2)).
 *   query[i] : FFN (+LN) of the query path: eq. (3) for i = 0, eq. (7) for i >= 1.  The pages use
 *              the same symbol SwiGLUFFN(i) for both; pass the hist[i] pointers for that reading.
 *   WQ, WK, WV, WO[i] : d x d; head j owns columns j*d_h .. (j+1)*d_h - 1 of WQ, WK, WV.
 *   WC[i]    : (i+1)d x d for i >= 1, row blocks ordered [o(1); ...; o(i); x_t]; WC[0] unused. */
typedef struct {
  stca_ffn hist[STCA_MAX_M];
  stca_ffn query[STCA_MAX_M];
  const void *WQ[STCA_MAX_M], *WK[STCA_MAX_M], *WV[STCA_MAX_M], *WO[STCA_MAX_M];
  const void *WC[STCA_MAX_M];
} stca_weights;

/* A ragged request-level batch: user u owns history rows hist_off[u] .. hist_off[u+1]-1 and
 * target rows tgt_off[u] .. tgt_off[u+1]-1 (the segment index tensor of ragged target attention). */
typedef struct {
  int32_t n_users;
  const int64_t *hist_off; /* n_users + 1 entries (device) */
  const int64_t *tgt_off;  /* n_users + 1 entries (device) */
  int64_t total_L;         /* [host] hist_off[n_users] */
  int64_t total_T;         /* [host] tgt_off[n_users] */
  int64_t max_L;           /* [host] largest per-user history length (an upper bound is fine) */
  int64_t max_T;           /* [host] largest per-user target count (an upper bound is fine) */
} stca_batch;

/* Workspace sizes in bytes (host only, no device work).  Return STCA_OK or an argument error. */
STCA_API int stca_encode_workspace_size(const stca_dims *dims, int64_t n_rows, size_t *bytes);
STCA_API int stca_attend_workspace_size(const stca_dims *dims, const stca_batch *batch, size_t *bytes);
STCA_API int stca_forward_workspace_size(const stca_dims *dims, const stca_batch *batch, size_t *bytes);
STCA_API int stca_predict_workspace_size(const stca_dims *dims, int64_t n_targets, size_t *bytes);

/* eq. (2): Xt[n_rows x d] = LN(SwiGLUFFN(X[n_rows x d])) with the weights of `ffn`
 * (gamma/beta required).  X and Xt are dims->dtype.  Rows are independent tokens. */
STCA_API int stca_encode(const stca_dims *dims, const stca_ffn *ffn, int64_t n_rows, const void *X, void *Xt,
                void *workspace, size_t workspace_bytes, void *stream);

/* eqs. (13), (6) for layer `layer` (0-based): given the layer's encoded history Xt
 * (total_L x d, dims->dtype) and the queries q (total_T x d, fp32), writes
 * o (total_T x d, fp32): each target attends only to its own user's history segment. */
STCA_API int stca_attend(const stca_dims *dims, const stca_weights *w, int32_t layer, const stca_batch *batch,
                const void *Xt, const float *q, float *o, void *workspace, size_t workspace_bytes,
                void *stream);

/* stca_attend without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same kernels
 * work in a fixed scratch array of 64 MiB per GPU that the library's code object holds, so the call
 * makes no allocation of any kind.  A batch whose stca_attend_workspace_size exceeds 64 MiB is
 * refused with STCA_E_WORKSPACE before any work.  Every call on one GPU uses that GPU's one array:
 * calls that overlap on a GPU (on different streams or host threads) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the array needs clearing between calls
 * (each call writes every scratch value before it reads it).  Otherwise as stca_attend. */
STCA_API int stca_attend_noalloc(const stca_dims *dims, const stca_weights *w, int32_t layer,
                                 const stca_batch *batch, const void *Xt, const float *q, float *o, void *stream);

/* eqs. (2)-(8): the whole stack.  X: total_L x d, xt: total_T x d (dims->dtype);
 * Z: total_T x M x d fp32, Z[t][i] = o(i+1) of target t. */
STCA_API int stca_forward(const stca_dims *dims, const stca_weights *w, const stca_batch *batch, const void *X,
                 const void *xt, float *Z, void *workspace, size_t workspace_bytes, void *stream);

/* eq. (9) of "Make It Long, Keep It Fast" (notes page, section 2.1, prediction head): the
 * prediction token z = SwiGLUFFN([o(1) || ... || o(M) || x_t] W_Z) of every target.
 *   WZ:  (M+1)d x d, row-major, dims->dtype; row blocks ordered [o(1); ...; o(M); x_t].
 *   ffn: the prediction FFN's W_u, W_v (d x rd) and W_o (rd x d), dims->dtype.  No LayerNorm
 *        follows (none is printed), so gamma/beta are not read and may be NULL.
 *   Z:   n_targets x M x d fp32 as written by stca_forward (Z[t][i] = o(i+1)).
 *   xt:  n_targets x d, dims->dtype.
 *   z:   n_targets x d fp32 (output).
 * Same conventions as the calls above; n_targets = 0 is a no-op. */
STCA_API int stca_predict(const stca_dims *dims, const void *WZ, const stca_ffn *ffn, int64_t n_targets,
                          const float *Z, const void *xt, float *z, void *workspace, size_t workspace_bytes,
                          void *stream);

/* ---- backward pass ---------------------------------------------------------------------------
 * Gradients of the forward of eqs. (2)-(8) (the training step of "Make It Long, Keep It Fast",
 * notes page, section 2.2: the stack is trained end to end with the loss of eq. (14), which is
 * outside this library) for an upstream gradient dZ of its output.  With L = sum(dZ * Z), the
 * call returns dL/dX, dL/dx_t and dL/dW for every weight slot, in fp32:
 *   - the history FFN of layer i (hist[i]) and the query FFN of layer i (query[i]) are separate
 *     slots even where they point at the same matrices; a caller sharing them adds the two;
 *   - every output is overwritten (not accumulated); gradients of query[i].gamma/beta for i >= 1
 *     without dims->query_ln are zeros; pointers may be NULL to skip dX, dxt and those unused
 *     query LayerNorm slots, every other gradient pointer is required;
 *   - the forward is recomputed inside the call in fp32 from the stored X, x_t and weights
 *     (dims->dtype storage; no bf16 rounding of intermediates), so results are the fp32
 *     gradients of the fp32 forward;
 *   - reductions over rows (tokens, targets) run in a fixed order: results are deterministic.
 * Memory: the workspace holds the encoded history of every layer in fp32 (M total_L d floats),
 * two buffers of per-user attention scores (h min(max_T total_L, max_L total_T) + 3 h total_T floats
 * each) and per-target intermediates; stca_backward_workspace_size gives the exact figure. */
typedef struct {
  float *dWu, *dWv; /* d x rd */
  float *dWo;       /* rd x d */
  float *dgamma, *dbeta; /* d */
} stca_ffn_grad;

typedef struct {
  float *dX;  /* total_L x d, or NULL */
  float *dxt; /* total_T x d, or NULL */
  stca_ffn_grad hist[STCA_MAX_M];
  stca_ffn_grad query[STCA_MAX_M];
  float *dWQ[STCA_MAX_M], *dWK[STCA_MAX_M], *dWV[STCA_MAX_M], *dWO[STCA_MAX_M]; /* d x d */
  float *dWC[STCA_MAX_M]; /* (i+1)d x d for i >= 1; dWC[0] unused */
} stca_grads;

STCA_API int stca_backward_workspace_size(const stca_dims *dims, const stca_batch *batch, size_t *bytes);
/* A larger workspace, at least this size, lets stca_backward keep the history FFN's intermediates from its
 * forward recompute (A = X W_u, G = X W_v and the pre-LayerNorm rows of every layer: 4 M total_L (2 rd + d)
 * bytes more) instead of computing them a second time for the derivative of eq. (2).  Same results up to
 * fp32 rounding order; the call picks the mode from workspace_bytes. */
STCA_API int stca_backward_workspace_size_keep(const stca_dims *dims, const stca_batch *batch, size_t *bytes);

/* X: total_L x d, xt: total_T x d (dims->dtype), dZ: total_T x M x d fp32 (the layout of Z in
 * stca_forward), grads: output pointers as described above (device).  Same conventions as the
 * forward: argument errors before any work, asynchronous on `stream`; a user with an empty
 * history gets NaN gradients. */
STCA_API int stca_backward(const stca_dims *dims, const stca_weights *w, const stca_batch *batch, const void *X,
                           const void *xt, const float *dZ, const stca_grads *grads, void *workspace,
                           size_t workspace_bytes, void *stream);

/* ---- stochastic-length training batches -----------------------------------------------------
 * "Make It Long, Keep It Fast" (notes page, length extrapolation: stochastic length sampling,
 * eqs. (15)-(17); element selection; batch-level load balancing, two steps).  A training batch
 * gives each user a random length L_train (a Beta draw mapped by eq. (16), aligned to 8), keeps
 * the user's most recent L_train history rows (the temporal suffix), truncates sequences so the
 * batch holds at most B * L_avg tokens, and lays the rows end to end with no padding; the
 * segment offsets are the index tensor the ragged kernels above take as hist_off. */
typedef struct {
  int32_t L_min;   /* shortest training length, >= 1 */
  int32_t L_max;   /* longest training length, L_min < L_avg < L_max */
  int32_t L_avg;   /* mean training length; the batch budget is n_users * L_avg tokens */
  int32_t L_infer; /* histories are first truncated to their most recent L_infer rows, >= 1 */
} stca_sl_params;

/* eq. (17): the Beta shape beta = alpha (L_max - L_avg) / (L_avg - L_min) that puts the mean of
 * eq. (16) at L_avg (alpha > 0).  Host only. */
STCA_API int stca_sl_beta(const stca_sl_params *p, double alpha, double *beta);

/* Host only: the lengths and segment offsets of a stochastic-length batch of n_users users.
 *   full_len [host]: n_users history lengths (>= 0) of the users' full histories.
 *   s        [host]: n_users draws in [0, 1] (the caller's Beta(alpha, beta) variates).
 *   order    [host]: a permutation of 0 .. n_users-1, the order in which sequences are truncated.
 *   len      [host, out]: n_users training lengths; hist_off [host, out]: n_users + 1 offsets.
 * Steps: L = L_min + s (L_max - L_min) (eq. (16)); rounded to the nearest multiple of 8 (halves
 * up) and clamped to [8 ceil(L_min/8), 8 floor(L_max/8)]; capped by min(full_len, L_infer); then,
 * while the total exceeds n_users * L_avg, sequences are shortened in `order`, each by as much of
 * the excess as it can give without going below 8 ceil(L_min/8), so the total equals that budget.  Returns STCA_E_ARG on bad
 * parameters, draws outside [0, 1] or an `order` that is not a permutation. */
STCA_API int stca_sl_plan(const stca_sl_params *p, int32_t n_users, const int64_t *full_len, const double *s,
                          const int32_t *order, int64_t *len, int64_t *hist_off);

/* Device: gathers the temporal suffix of every user into X_packed (total x d, dims->dtype, no
 * padding): packed row hist_off[u] + j is full-history row full_off[u+1] - len[u] + j.
 *   full_off: n_users + 1 offsets of the full histories in X_full (device);
 *   hist_off: n_users + 1 offsets of the packed batch (device), as from stca_sl_plan, with
 *             hist_off[u+1] - hist_off[u] <= full_off[u+1] - full_off[u];
 *   total:    [host] hist_off[n_users];
 *   max_len:  [host] an upper bound on hist_off[u+1] - hist_off[u] (the largest length of the plan).
 * Only dims->d and dims->dtype are read.  Asynchronous on `stream`. */
STCA_API int stca_sl_pack(const stca_dims *dims, int32_t n_users, const int64_t *full_off, const int64_t *hist_off,
                          int64_t total, int64_t max_len, const void *X_full, void *X_packed, void *stream);

/* ---- local same-ID token merging (LITM) -----------------------------------------------------
 * "TM20K：老师读全文，学生读缩写" (notes page, section 4.2.1; the threshold T of section 5.4, the
 * host/device split of section 4.1): tokens of a history that carry the same key (item) ID and
 * sit at most T positions apart are summed into one token, a local merge rather than a
 * deduplication of the whole sequence.  Reading of the page where it is silent: positions are
 * scanned in order and token p joins the group of the latest earlier token of its user with the
 * same ID when that token is at most T positions back, otherwise it opens a group; a group is
 * placed at its first token, so merged histories keep the order of first occurrences; tokens of
 * different users never merge. */

/* Host only.  Groups of a batch of n_users histories.
 *   hist_off   [host]: n_users + 1 nondecreasing offsets, hist_off[0] = 0 (total = hist_off[n_users]).
 *   item_id    [host]: total item IDs, one per history row.
 *   T: largest position gap that still merges (>= 0; 0 merges nothing).
 *   merged_off [host, out]: n_users + 1 offsets of the merged histories (in groups).
 *   group_off  [host, out]: n_groups + 1 offsets into members (room for total + 1 entries).
 *   members    [host, out]: the total source rows, grouped, in position order within a group.
 *   n_groups   [host, out]: number of groups (merged rows).
 * Returns STCA_E_ARG on NULL pointers, T < 0, n_users < 0 or offsets that are not as stated. */
STCA_API int stca_litm_plan(int32_t n_users, const int64_t *hist_off, const int64_t *item_id, int32_t T,
                            int64_t *merged_off, int64_t *group_off, int64_t *members, int64_t *n_groups);

/* Device: X_merged[g] = sum of the rows X[members[j]], group_off[g] <= j < group_off[g+1], for the
 * n_groups groups of a plan (group_off, members: device copies of the plan's arrays).  X is
 * n_rows x d and X_merged n_groups x d, both dims->dtype; sums run in fp32 in member order and
 * are rounded once to the storage type.  Member indices outside [0, n_rows) are skipped.
 * 16-byte aligned rows; n_groups = 0 is a no-op. */
STCA_API int stca_litm_merge(const stca_dims *dims, int64_t n_rows, int64_t n_groups, const int64_t *group_off,
                             const int64_t *members, const void *X, void *X_merged, void *stream);

/* ---- per-kernel timing (HIP events on the call's stream) ---------------------------------- */
typedef struct stca_profiler stca_profiler; /* opaque, host-side; not thread-safe */

enum {
  STCA_PHASE_PACK = 0,   /* weight re-layout for the MFMA encode */
  STCA_PHASE_ENCODE,     /* history encode, eq. (2) (one launch per layer) */
  STCA_PHASE_QUERY,      /* query path, eqs. (3), (7) */
  STCA_PHASE_UPROJ,      /* u = (q W_Q) W_K^T, eq. (13) */
  STCA_PHASE_ATTEND,     /* split-L attention over the history (one launch per layer) */
  STCA_PHASE_COMBINE,    /* merge of split-L partial softmax states */
  STCA_PHASE_PROJECT,    /* (alpha X~) W_V and W_O, eqs. (13), (6) */
  STCA_PHASE_BWD_RECOMPUTE, /* backward: fp32 encode of the history for every layer, eq. (2) */
  STCA_PHASE_BWD_ATTEND,    /* backward: softmax statistics, query- and key-side derivative kernels */
  STCA_PHASE_BWD_ENCODE,    /* backward: derivative of eq. (2) over the history rows (per layer) */
  STCA_PHASE_BWD_TARGET,    /* backward: every per-target step (query path, projections, W_C) */
  STCA_N_PHASES
};

typedef struct {
  double ms[STCA_N_PHASES];      /* summed elapsed milliseconds per phase since the last reset */
  int64_t launches[STCA_N_PHASES];
} stca_profile_report;

STCA_API int stca_profiler_create(stca_profiler **out);
STCA_API int stca_profiler_destroy(stca_profiler *p);
STCA_API int stca_profiler_reset(stca_profiler *p);
/* Waits for the recorded events to complete, then sums them (host blocks; the device is not synced). */
STCA_API int stca_profiler_read(stca_profiler *p, stca_profile_report *out);
/* stca_forward with an event pair recorded around every phase launch (prof may be NULL). */
STCA_API int stca_forward_profiled(const stca_dims *dims, const stca_weights *w, const stca_batch *batch,
                          const void *X, const void *xt, float *Z, void *workspace,
                          size_t workspace_bytes, void *stream, stca_profiler *prof);

/* stca_backward with an event pair recorded around every phase (prof may be NULL). */
STCA_API int stca_backward_profiled(const stca_dims *dims, const stca_weights *w, const stca_batch *batch,
                                    const void *X, const void *xt, const float *dZ, const stca_grads *grads,
                                    void *workspace, size_t workspace_bytes, void *stream, stca_profiler *prof);

/* ---- graph replay of the forward -------------------------------------------------------------
 * A forward over a small batch is a few dozen short kernels, and launch overhead dominates it.
 * stca_forward_graph_create records one stca_forward with exactly these arguments (the device
 * pointers and the batch sizes are baked in) as a HIP graph; stca_graph_launch replays it on
 * `stream`.  A replay reads whatever the buffers hold at that time, so new inputs of the same
 * shapes in the same buffers need no new graph.  The graph owns driver resources (released by
 * stca_graph_destroy), not device memory: the workspace stays the caller's and must stay valid
 * and unused by other work while a replay runs.  Argument errors are returned as by
 * stca_forward, before anything is recorded.  Capture happens on a stream of the library's own;
 * nothing runs on the device until the first launch. */
typedef struct stca_graph stca_graph; /* opaque, host-side */
STCA_API int stca_forward_graph_create(const stca_dims *dims, const stca_weights *w, const stca_batch *batch,
                                       const void *X, const void *xt, float *Z, void *workspace,
                                       size_t workspace_bytes, stca_graph **out);
STCA_API int stca_graph_launch(stca_graph *g, void *stream);
STCA_API int stca_graph_destroy(stca_graph *g); /* NULL is a no-op */

/* ---- batch check (debug) -----------------------------------------------------------------------
 * Checks the device offsets of `batch` against its host fields and writes to *result (a device
 * int32) the OR of the conditions it breaks, 0 for a batch that meets the contract.  Asynchronous
 * on `stream`; read *result after the stream has reached the call.  Host argument errors are
 * returned before any work, as for the other calls. */
enum {
  STCA_BATCH_BAD_START = 1,       /* hist_off[0] or tgt_off[0] is not 0 */
  STCA_BATCH_BAD_END = 2,         /* hist_off[n_users] != total_L or tgt_off[n_users] != total_T */
  STCA_BATCH_DECREASING = 4,      /* an offset array decreases */
  STCA_BATCH_OVER_MAX_L = 8,      /* a user has more than max_L history rows */
  STCA_BATCH_OVER_MAX_T = 16,     /* a user has more than max_T targets */
  STCA_BATCH_EMPTY_HISTORY = 32   /* a user with targets has no history (allowed: NaN outputs) */
};
STCA_API int stca_validate_batch(const stca_batch *batch, int32_t *result, void *stream);

/* ---- index checks of the debug build --------------------------------------------------------
 * A library built with STCA_DEBUG_BOUNDS defined (libstca_debug.so next to libstca.so) checks, in
 * its kernels, the indices that ragged offsets and workspace plans drive (history tile rows
 * against the work item's chunk, output and partial-state rows against their buffers, work items
 * against the list's capacity, padded operand rows against their strides).  A failed check never
 * faults: it sets a bit in a device word and the kernel runs on.  stca_debug_flags synchronises the
 * device, writes the OR of the bits recorded since the last clear to *flags (STCA_DBG_* below) and
 * clears them if `clear` is nonzero; *checks_enabled (may be NULL) is 1 in the debug build and 0 in
 * the ordinary one, where *flags is always 0 and no device work is done.  stca_debug_selftest
 * records STCA_DBG_SELFTEST from a kernel on `stream` (debug build; a no-op otherwise), to show the
 * mechanism reports what it records. */
enum {
  STCA_DBG_ATTEND_RANGE = 1,     /* a work item's history range outside [0, total_L] */
  STCA_DBG_ATTEND_FETCH = 2,     /* a history tile row outside the item's chunk */
  STCA_DBG_ATTEND_OUT = 4,       /* an attention output row past total_T * h */
  STCA_DBG_ATTEND_PART = 8,      /* a partial-state row past the workspace's partial rows */
  STCA_DBG_COMBINE_PART = 16,    /* the combine reading partial rows past the workspace's */
  STCA_DBG_WORKLIST = 32,        /* a work item written past the list's capacity */
  STCA_DBG_GEMM_PAD = 64,        /* a transposed backward operand's row chunk past its row stride */
  STCA_DBG_SELFTEST = (int)0x80000000u
};
STCA_API int stca_debug_flags(uint32_t *flags, int32_t *checks_enabled, int32_t clear);
STCA_API int stca_debug_selftest(void *stream);

/* ---- diagnostics ---------------------------------------------------------------------------- */
STCA_API const char *stca_status_string(int status);
STCA_API const char *stca_last_error(void); /* thread-local detail of the last failure in this thread */
STCA_API const char *stca_version(void);

#ifdef __cplusplus
}
#endif
#endif /* STCA_H */
