/*
 * xattn - one-history-to-many-candidates cross-attention on AMD Instinct
 * MI355X (gfx950).  C ABI.
 *
 * What it computes.  A batch holds R requests.  Request r owns L_r memory rows
 * (its shared history) and N_r candidates; every candidate carries q query
 * tokens.  For query row `row = c*q + s` of candidate c in request r (slot s):
 *
 *     Q[row]          = Z[row] . W_Q[s]                              (TSP)
 *     O[row, head h]  = softmax( Q_h K_r,h^T / sqrt(d_h) ) V_r,h       (Eq. 7)
 *
 * with heads splitting the d feature columns contiguously, d_h = d / heads.
 * Sources (the pages on the subject):
 *   - ReST reading note (paper-archivist), s.3.3.1 Eq. (7): projection-free
 *     K/V - the encoder output H is used as both K and V, so per-candidate
 *     work has no W_K / W_V.  The output gate and W_o of Eq. (7) are left to
 *     the caller: O is the concatenated multi-head attention output.
 *   - ReST reading note, s.3.3.2 Eq. (8): token-specific parameterisation -
 *     each query-token type (slot) s has its own W_Q[s].
 *   - ReST reading note, s.3.5: shared-prefix serving - H is computed once per
 *     request and all N candidates' query tokens are decoded against it.
 *   - TransX technical report (paper-daily), s.2: a compact behaviour memory
 *     turned into separate keys and values that every candidate's query
 *     cross-attends (XATTN_KV_SEPARATE).
 *   - HELIX card (ai-papers-daily, "Sequence Modeling"): candidate-independent
 *     KV cache, candidate side does cross-attention only, padding-free
 *     variable-length execution (the ragged cu_* offsets below).
 *
 * Conventions.
 *   - Every tensor is row-major, device-resident and owned by the caller.
 *     Element type is bf16 (XATTN_BF16) or fp32 (XATTN_FP32) for Z, W_Q, K, V
 *     and O alike; offsets are int32.
 *   - Z     [total_cand][q][d]   query tokens; row c*q+s is slot s of cand c.
 *   - W_Q   [q][d][d]            output-major: W_Q[s][o][i] multiplies Z[.][i]
 *                                into Q[.][o] (W_Q[s] of Eq. (7) transposed,
 *                                the layout of a PyTorch Linear weight).
 *   - K     [total_kv][d]        memory rows; this is H in XATTN_KV_SHARED.
 *   - V     [total_kv][d]        values (XATTN_KV_SEPARATE); must be NULL in
 *                                XATTN_KV_SHARED, where V = K = H.
 *   - cu_seqlens_kv [R+1]        cu[0] = 0, non-decreasing, cu[R] = total_kv;
 *                                request r's memory rows are
 *                                [cu_seqlens_kv[r], cu_seqlens_kv[r+1]).
 *   - cu_cand       [R+1]        cu[0] = 0, non-decreasing,
 *                                cu[R] = total_cand; request r's candidates.
 *   - O     [total_cand][q][d]   output, heads concatenated by column.
 *   - A request with L_r = 0 gets all-zero output rows (the pages route users
 *     without memory to a fallback model; zero is this library's convention).
 *     A request with N_r = 0 produces no rows.  No mask: every query row
 *     attends to all L_r rows of its request (xattn_forward_prefix limits
 *     each candidate to a prefix of them).
 *   - Precision: XATTN_BF16 multiplies bf16 operands into fp32 accumulators
 *     on the matrix cores; Q is rounded to bf16 after the projection and once
 *     more after scaling by log2(e)/sqrt(d_h) (the softmax scale folded into
 *     the query operands) - except on the short-memory path
 *     (XATTN_PATH_SHORT), which rounds Q once and scales the fp32 scores; the
 *     softmax weights are rounded to bf16 for the PV product; O is rounded to
 *     bf16 (nearest-even).  XATTN_FP32 computes in fp32 throughout.
 *
 * Supported: d_h = d / heads in {32, 64, 128} for bf16 (1..128 for fp32),
 * q in [1, 64], d a multiple of 32 for bf16, R >= 0.
 *
 * Errors.  Every entry point returns an xattn_status.  Problems visible on
 * the host (NULL pointers, bad sizes, unsupported shapes, a workspace that is
 * too small) return before anything is enqueued.  Launch failures return
 * XATTN_EHIP.  xattn_last_error() describes the last failure on the calling
 * thread.  The device re-checks the offset arrays (cu[0] = 0, non-decreasing,
 * cu[R] equal to the totals passed on the host) before any kernel reads
 * through them; on a mismatch it computes nothing and raises a flag in the
 * workspace that xattn_device_error() reads back.
 *
 * Streams and threads.  Work is enqueued on `stream` (a hipStream_t; NULL is
 * the default stream) and returns without synchronising.  A context may be
 * used from one thread at a time; separate contexts are independent.  The
 * workspace must not be shared by calls that may run concurrently.  No entry
 * point except xattn_create / xattn_destroy allocates or frees memory.
 */
#ifndef XATTN_H
#define XATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct xattn_ctx xattn_ctx;

typedef enum {
    XATTN_OK = 0,
    XATTN_EINVAL = -1,        /* invalid argument; nothing enqueued            */
    XATTN_EUNSUPPORTED = -2,  /* valid but not supported (e.g. d_h = 48, bf16) */
    XATTN_EHIP = -3,          /* HIP runtime error                             */
    XATTN_EWORKSPACE = -4,    /* workspace NULL or smaller than required       */
    XATTN_EDEVICE_VALIDATION = -5  /* xattn_device_error: the device found the
                                      offset arrays inconsistent with the host
                                      totals (nothing was computed)          */
} xattn_status;

typedef enum { XATTN_BF16 = 0, XATTN_FP32 = 1 } xattn_dtype;

typedef enum {
    XATTN_KV_SHARED = 0,   /* K = V = H, projection-free (ReST Eq. (7))       */
    XATTN_KV_SEPARATE = 1  /* separate K and V memory (TransX behaviour memory) */
} xattn_kv_mode;

typedef struct {
    int32_t d_model;        /* d: model width (query, key and value width)   */
    int32_t n_slots;        /* q: query tokens per candidate (TSP slots)      */
    xattn_dtype dtype;
    xattn_kv_mode kv_mode;
    int32_t device;         /* HIP device ordinal the context launches on     */
} xattn_config;

/* Create a context.  Validates cfg (d_model >= 1, 1 <= n_slots <= 64, known
 * dtype and kv_mode, device >= 0) and copies it; allocates only the handle.
 * Returns XATTN_EINVAL (and *out = NULL) on a bad config. */
xattn_status xattn_create(const xattn_config* cfg, xattn_ctx** out);

/* Destroy a context created by xattn_create.  NULL is allowed. */
void xattn_destroy(xattn_ctx* ctx);

/* Bytes of device workspace xattn_forward needs for a batch of
 * `num_requests` requests, `total_cand` candidates and `heads` heads: a plan
 * header, one 16-byte work item per query tile, and the projected queries
 * (total_cand * q * d elements of the context's type).  Returns 0 on invalid
 * arguments. */
size_t xattn_workspace_size(const xattn_ctx* ctx, int32_t num_requests,
                            int32_t total_cand, int32_t heads);

/* Shared-history cross-attention forward (Eq. (7) attention with Eq. (8)
 * per-slot W_Q; layouts and precision in the header comment).  Enqueues on
 * `stream` one of (xattn_forward_path() tells which):
 *   - one kernel - bf16 batches of at most 16 requests on a model of at most
 *     256 features: the attention kernel plans the batch, projects its own
 *     queries and writes the plan into the workspace;
 *   - one short-memory kernel, which plans the batch (in request order),
 *     projects and attends in one launch and writes the plan into the
 *     workspace - bf16 batches on a 256-feature model whose memories are
 *     short on average (total_kv <= 96 * num_requests with separate K and V,
 *     192 * num_requests with K = V; the TransX behaviour memory, TransX
 *     report s.2); any single memory may be longer;
 *   - the TSP projection (whose launch also runs the varlen planner in one
 *     extra work-group) and then the attention kernel, which reads the
 *     projected queries and the plan from the workspace.
 * The three compute the same roundings (below).
 * `workspace` is device memory of at least xattn_workspace_size() bytes,
 * owned by the caller; its contents on entry are ignored.
 * Errors: XATTN_EINVAL for NULL pointers / negative counts / heads not
 * dividing d / V given in shared mode or missing in separate mode;
 * XATTN_EUNSUPPORTED for an unsupported d_h; XATTN_EWORKSPACE for a small
 * workspace; XATTN_EHIP for a launch failure. */
xattn_status xattn_forward(xattn_ctx* ctx,
                           const void* Z, const void* W_Q,
                           const void* K, const void* V,
                           const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                           int32_t num_requests, int32_t total_cand,
                           int32_t total_kv, int32_t heads,
                           void* O, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Bytes of the device scratch array that xattn_forward_noalloc uses in place
 * of a workspace (32 MiB).  Every GPU the library runs on holds one such
 * array from the first xattn_forward_noalloc call on it until the process
 * ends. */
#define XATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

/* xattn_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same computation, kernels, launches and results as xattn_forward; the
 * workspace is replaced by a library-owned device array of
 * XATTN_NOALLOC_SCRATCH_BYTES per GPU.  No HIP allocation, free or memset is
 * made: the call validates, makes ctx's device current, looks up (first call
 * on that device: resolves) the array's device address, and enqueues the
 * kernels on `stream`.
 *   - Scratch use: the plan (a 256-byte header and 16 bytes per query tile,
 *     at most q * ceil-sum of N_r / 32 tiles) on the single-launch and
 *     short-memory paths; on the other paths (projection GEMM + attention,
 *     fp32) also the projected queries, total_cand * q * d elements of the
 *     context's type, after the plan (256-byte aligned).  A batch whose path
 *     needs more than XATTN_NOALLOC_SCRATCH_BYTES is rejected with
 *     XATTN_EUNSUPPORTED before anything is enqueued (use xattn_forward).
 *   - Nothing in the array needs to start at zero: every call rewrites the
 *     plan header before any kernel reads it.
 *   - All calls on one GPU share that GPU's array and it keeps the last
 *     call's contents: calls that may overlap on one GPU (other streams,
 *     other threads, other contexts) race on it and must be serialised by
 *     the caller.
 *   - The device-side check of the offset arrays still runs (on a mismatch
 *     no output is computed), but its flag stays in the library's array;
 *     callers that need to read it use xattn_forward and xattn_device_error.
 * Other arguments and errors as for xattn_forward; a HIP failure while
 * resolving the array's address is XATTN_EHIP. */
xattn_status xattn_forward_noalloc(xattn_ctx* ctx,
                                   const void* Z, const void* W_Q,
                                   const void* K, const void* V,
                                   const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                                   int32_t num_requests, int32_t total_cand,
                                   int32_t total_kv, int32_t heads,
                                   void* O, void* stream);

/* xattn_forward with a per-candidate memory prefix (ReST reading note, s.3.5:
 * under the unified-long-term reading every training sample of a user sees
 * only the part of that user's sequence that precedes it, so the candidates
 * of one request may see different prefixes of the shared memory).
 *   - cand_kv_len [total_cand] int32, device: candidate c of request r
 *     attends to memory rows [cu_seqlens_kv[r], cu_seqlens_kv[r] + n) with
 *     n = cand_kv_len[c] clamped to [0, L_r]; every slot of the candidate
 *     uses the same n.  A candidate with n = 0 gets all-zero output rows.
 * In bf16, one launch for a batch of at most 16 requests on a model of at
 * most 256 features (the attention kernel plans the batch, projects its own
 * queries and applies the per-row mask, as xattn_forward's single launch
 * does), otherwise two (projection GEMM with the planner, then the attention
 * kernel with the per-row mask); the short-memory kernel is never used here.
 * Three launches in fp32.  Other arguments,
 * workspace and errors as for xattn_forward; a NULL cand_kv_len with
 * total_cand > 0 is XATTN_EINVAL.  With every cand_kv_len[c] >= L_r the
 * result equals xattn_forward's. */
xattn_status xattn_forward_prefix(xattn_ctx* ctx,
                                  const void* Z, const void* W_Q,
                                  const void* K, const void* V,
                                  const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                                  const int32_t* cand_kv_len,
                                  int32_t num_requests, int32_t total_cand,
                                  int32_t total_kv, int32_t heads,
                                  void* O, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Training forward: xattn_forward (cand_kv_len NULL) or xattn_forward_prefix
 * (cand_kv_len not NULL) that also stores, for xattn_backward_saved, the
 * softmax normaliser of every query row and head (ReST reading note s.3.3.1,
 * Eq. (7): the denominator of the row's softmax over its request's memory).
 *   - lse [total_cand][q][heads] fp32, device, written: the base-2 logarithm
 *     of sum_j exp(q_h . k_{h,j} / sqrt(d_h)) over the rows j the row sees,
 *     with q_h the bf16 projected query as the products use it: scaled by
 *     log2(e)/sqrt(d_h) and rounded to bf16 once more - except on the
 *     short-memory path (XATTN_PATH_SHORT), whose products use the query
 *     rounded once and scale the fp32 scores, so its lse belongs to those
 *     scores (xattn_backward_saved recomputes with the pre-scaled query, so
 *     there the weights it forms sum to 1 only up to that rounding); -inf for
 *     a row that sees no memory.
 * O, the workspace, the launches and the other arguments as for
 * xattn_forward (or xattn_forward_prefix).  bf16 contexts only
 * (XATTN_EUNSUPPORTED otherwise); a NULL lse with total_cand > 0 is
 * XATTN_EINVAL. */
xattn_status xattn_forward_train(xattn_ctx* ctx,
                                 const void* Z, const void* W_Q,
                                 const void* K, const void* V,
                                 const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                                 const int32_t* cand_kv_len,
                                 int32_t num_requests, int32_t total_cand,
                                 int32_t total_kv, int32_t heads,
                                 void* O, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Projection and attention without re-planning (one kernel where
 * xattn_forward would run one): like xattn_forward, but the plan is read
 * from `workspace`, where a previous xattn_plan or xattn_forward call left it
 * for the SAME offsets and shape arguments (a decoder with
 * several cross-attention layers over one batch plans once and runs the
 * projection and attention per layer).  Arguments and errors as for
 * xattn_forward.  If the workspace holds the plan of a different batch shape
 * (another candidates-per-tile size), the attention kernel computes nothing;
 * a plan of a different batch with the same tile size gives undefined
 * output. */
xattn_status xattn_attend(xattn_ctx* ctx,
                          const void* Z, const void* W_Q,
                          const void* K, const void* V,
                          const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                          int32_t num_requests, int32_t total_cand,
                          int32_t total_kv, int32_t heads,
                          void* O, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Attention kernel alone, over queries the caller already projected:
 * Q [total_cand][q][d] in the context's type holds Z . W_Q[slot] (as
 * xattn_project writes it); the plan is read from `workspace` as for
 * xattn_attend.  For callers that fuse the query projection into their own
 * producer.  Errors as for xattn_forward (NULL Q is XATTN_EINVAL). */
xattn_status xattn_attend_q(xattn_ctx* ctx, const void* Q,
                            const void* K, const void* V,
                            const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                            int32_t num_requests, int32_t total_cand,
                            int32_t total_kv, int32_t heads,
                            void* O, void* workspace, size_t workspace_bytes,
                            void* stream);

/* xattn_attend_q with the per-candidate memory prefix of
 * xattn_forward_prefix: attention over caller-projected queries Q, the plan
 * read from `workspace` (left there by xattn_forward_prefix, xattn_forward or
 * xattn_plan for the same batch), candidate c limited to the first
 * cand_kv_len[c] memory rows of its request (clamped to [0, L_r]).  Errors as
 * for xattn_attend_q; a NULL cand_kv_len with total_cand > 0 is
 * XATTN_EINVAL. */
xattn_status xattn_attend_q_prefix(xattn_ctx* ctx, const void* Q,
                                   const void* K, const void* V,
                                   const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                                   const int32_t* cand_kv_len,
                                   int32_t num_requests, int32_t total_cand,
                                   int32_t total_kv, int32_t heads,
                                   void* O, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Bytes of device workspace xattn_backward needs for this batch shape (0 on
 * invalid arguments). */
size_t xattn_backward_workspace_size(const xattn_ctx* ctx, int32_t num_requests,
                                     int32_t total_cand, int32_t total_kv, int32_t heads);

/* Backward pass of xattn_forward: the gradients of <dO, O> with respect to
 * the query tokens, the per-slot W_Q and the memory, for the loss gradient
 * dO of the attention output O (ReST reading note s.3.3.1 Eq. (7) with
 * Eq. (8)'s per-slot W_Q).  The memory gradient of a request sums the
 * contributions of all its candidates' query rows: the candidates of one
 * user send their gradients back into the one encoded memory (TransX
 * report s.2, trajectory packing; ReST reading note s.3.5, ULT).
 *   - Z, W_Q, K, V, offsets, shapes: as for xattn_forward (the same batch).
 *   - dO  [total_cand][q][d] context type: gradient of the loss w.r.t. O.
 *   - dZ  [total_cand][q][d] context type.
 *   - dW_Q [q][d][d] fp32 in both modes, output-major like W_Q, summed over
 *     every candidate of every request (overwritten, not accumulated).
 *   - dK  [total_kv][d] context type.  In XATTN_KV_SHARED mode this is the
 *     gradient of H, which is both key and value (dV must be NULL).
 *   - dV  [total_kv][d] context type in XATTN_KV_SEPARATE mode.
 *   - cand_kv_len [total_cand] int32 or NULL: the per-candidate prefix of
 *     xattn_forward_prefix (the backward of that forward); NULL for the
 *     backward of xattn_forward.
 * Memory rows that no query row sees get zero gradient; requests without
 * memory rows give zero dZ.  The forward statistics (softmax normaliser and
 * <dO, O> per row and head) are recomputed inside; every reduction runs in a
 * fixed order, so the result is deterministic bit for bit.  Enqueues, on
 * `stream`: the projection (with the query-tile planner), the memory-tile
 * planner, the statistics pass, the dQ kernel, the dK/dV kernel, a weight
 * transpose, the dZ GEMM and the dW_Q kernels.  bf16: products on the matrix
 * cores with fp32 accumulation; P and dS are rounded to bf16 as operands,
 * dQ to bf16 before the dZ and dW_Q products.  `workspace` holds at least
 * xattn_backward_workspace_size() bytes.  Errors as for xattn_forward; NULL
 * dO, dZ, dW_Q or dK (where rows exist) is XATTN_EINVAL.  On offsets that
 * fail the device check nothing is written. */
xattn_status xattn_backward(xattn_ctx* ctx,
                            const void* Z, const void* W_Q,
                            const void* K, const void* V, const void* dO,
                            const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                            const int32_t* cand_kv_len,
                            int32_t num_requests, int32_t total_cand,
                            int32_t total_kv, int32_t heads,
                            void* dZ, float* dW_Q, void* dK, void* dV,
                            void* workspace, size_t workspace_bytes, void* stream);

/* (dO, and O where given, are read in 16-byte pieces: rows of d bf16
 * elements, so the base pointers must be 16-byte aligned - XATTN_EINVAL
 * otherwise, for both backward entry points.) */

/* xattn_backward from the statistics of xattn_forward_train: O
 * [total_cand][q][d] bf16 (16-byte aligned, as dO) and lse
 * [total_cand][q][heads] fp32 are that call's outputs for the same inputs
 * (and the same cand_kv_len).  The statistics pass (a repeat of the forward)
 * is replaced by one pass over dO and O for D = <dO_row, O_row> per head; D
 * is taken from the bf16 O rather than the forward's fp32 accumulators, so
 * the gradients differ from xattn_backward's by rounding.  Same workspace
 * size, outputs and errors as xattn_backward; bf16 contexts only
 * (XATTN_EUNSUPPORTED otherwise); NULL O or lse with total_cand > 0, or a
 * misaligned O or dO, is XATTN_EINVAL.  Stored statistics of other inputs
 * give undefined gradients. */
xattn_status xattn_backward_saved(xattn_ctx* ctx,
                                  const void* Z, const void* W_Q,
                                  const void* K, const void* V, const void* dO,
                                  const void* O, const float* lse,
                                  const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                                  const int32_t* cand_kv_len,
                                  int32_t num_requests, int32_t total_cand,
                                  int32_t total_kv, int32_t heads,
                                  void* dZ, float* dW_Q, void* dK, void* dV,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Coded memory (TransX technical report, s.3).  A published memory keeps,
 * for every row and head, the length of the head's key (or value) vector and
 * its direction rotated into the eigenbasis of the directions' covariance and
 * quantised coordinate by coordinate, with more bits for coordinates of more
 * energy under a fixed total.  The codebook (fitted offline on a sample of
 * memory vectors) is device data:
 *   rotation[h][o][i]  column i = i-th eigenvector of head h (fp32,
 *                      [heads][d_h][d_h]);
 *   bits[h][i]         bits of rotated coordinate i (uint8, 0..8), summing to
 *                      budget_bits for every head;
 *   center, half_range [heads][d_h] fp32: coordinate i is quantised
 *                      uniformly on [center - half, center + half] (mid-rise,
 *                      clamped; a coordinate with 0 bits reads as center).
 * Codes are packed least-significant bit first, coordinate 0 first, into
 * budget_bits/32 uint32 words per (row, head); codes [heads][rows][words],
 * norms [heads][rows] fp32 (head-major, so one head's tile is contiguous).
 * bf16 contexts only; d_h in {32, 64, 128}. */
typedef struct {
    int32_t budget_bits;      /* multiple of 32, at most 8 * d_h              */
    const uint8_t* bits;      /* [heads][d_h]                                 */
    const float* center;      /* [heads][d_h]                                 */
    const float* half_range;  /* [heads][d_h], > 0 where bits > 0             */
    const float* rotation;    /* [heads][d_h][d_h]                            */
} xattn_codebook;

/* Fit a codebook on the host from a calibration sample of memory rows
 * (TransX report s.3: the directions' covariance is estimated on a sample,
 * the rotation is its full eigenvector matrix, bits go by energy under a
 * fixed total).  Offline calibration, fp64 inside, all pointers host memory:
 *   - X [n_rows][d_model] fp32: the sample (key rows for a key codebook,
 *     value rows for a value codebook);
 *   - per head h, over the directions u = x_h / |x_h| of the rows with
 *     |x_h| > 0: mean mu and centred covariance C = E diag(lam) E^T, lam
 *     descending (ties keep their order), each column of E signed so that
 *     its largest-magnitude entry is positive;
 *   - outputs, layouts of xattn_codebook: rotation[h] = E (row-major,
 *     column i = eigenvector i), center[h] = E^T mu, half_range[h] =
 *     3 sqrt(max(lam, 0)), bits[h] = integers in [0, 8] summing to
 *     budget_bits, handed out one at a time to the largest lam_i 4^-b_i
 *     (lower index on ties).
 * Errors: XATTN_EINVAL for NULL pointers, n_rows < 1, heads not dividing
 * d_model, or a head whose sample slices are all zero; XATTN_EUNSUPPORTED
 * for budget_bits outside [0, 8 d_h].  Enqueues nothing. */
xattn_status xattn_codec_fit(int32_t d_model, int32_t heads, const float* X, int64_t n_rows,
                             int32_t budget_bits, uint8_t* bits, float* center,
                             float* half_range, float* rotation);

/* Encode memory rows X [n_rows][d] (bf16) with codebook cb into codes and
 * norms (layouts above).  The nearline publishing step. */
xattn_status xattn_codec_encode(xattn_ctx* ctx, const xattn_codebook* cb, int32_t heads,
                                const void* X, int32_t n_rows, uint32_t* codes, float* norms,
                                void* stream);

/* Query weights for a coded memory: W_Q_rot[s] = W_Q[s] with the rows of
 * head h replaced by rotation_h^T times them (output-major like W_Q, bf16),
 * so the projection delivers queries in the keys' rotated basis.  Weights
 * are static: fold once per codebook. */
xattn_status xattn_codec_fold_query_weights(xattn_ctx* ctx, const xattn_codebook* cb_k,
                                            int32_t heads, const void* W_Q, void* W_Q_rot,
                                            void* stream);

/* Bytes of device workspace xattn_forward_codec needs to decode the memory
 * once per call: xattn_workspace_size() plus one (shared mode) or two
 * (separate mode) bf16 planes of total_kv x d (0 on invalid arguments). */
size_t xattn_codec_workspace_size(const xattn_ctx* ctx, int32_t num_requests,
                                  int32_t total_cand, int32_t total_kv, int32_t heads);

/* xattn_forward over a coded memory: O[row, head h] = softmax(q_h k_h^T /
 * sqrt(d_h)) v_h with every k, v the decoded vector norm * rotation *
 * reconstruction.  With a workspace of xattn_codec_workspace_size() bytes
 * (and not the short path below): the memory is decoded once into bf16
 * planes in the workspace and xattn_forward's kernels run over them with
 * the queries projected over W_Q_rot.  Separate mode: keys in the rotated
 * basis, values rotated back.  Shared mode: one plane in the rotated basis
 * serves as key and value, and a last launch rotates the output rows back
 * (one more bf16 rounding of O).  With a workspace of only
 * xattn_workspace_size() bytes: two launches, the projection GEMM over
 * W_Q_rot (with the planner), then the attention kernel, which reconstructs
 * each memory tile while staging it in LDS (HBM carries codes and norms
 * only), accumulates in the rotated basis and rotates each output row back.  On a 256-feature
 * model with short memories (the xattn_forward short-path rule, at most 96
 * rows on average in both modes) they are the planner and the short-memory
 * kernel, which decodes each request's memory once per work-group (keys in
 * the rotated basis, values rotated back) and projects and attends as
 * xattn_forward's short path does.  Shared mode: the
 * memory is both key and value (cb_v, v_codes, v_norms NULL).  Separate mode:
 * cb_v with the same budget_bits as cb_k.  Offsets, shapes, workspace
 * (xattn_workspace_size) and errors as for xattn_forward; XATTN_EUNSUPPORTED
 * in fp32 mode or for a budget that is not a positive multiple of 32 at
 * most 8 * d_h. */
xattn_status xattn_forward_codec(xattn_ctx* ctx, const xattn_codebook* cb_k,
                                 const xattn_codebook* cb_v, const void* Z, const void* W_Q_rot,
                                 const uint32_t* k_codes, const float* k_norms,
                                 const uint32_t* v_codes, const float* v_norms,
                                 const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                                 int32_t num_requests, int32_t total_cand, int32_t total_kv,
                                 int32_t heads, void* O, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Varlen plan alone (integer outputs, for callers that want the row map and
 * for tests).  The pages pack ragged requests without padding (ReST reading
 * note s.5.5: padding removal; HELIX card, "Sequence Modeling": padding-free
 * variable-length execution; TransX report s.2: each request's memory goes to
 * that request's candidates); this is the work list of that packing.
 * Writes, on the device:
 *   cu_q[r]      = q * cu_cand[r]                (R+1 entries)
 *   row_req[row] = r for cu_q[r] <= row < cu_q[r+1]   (total_cand*q entries;
 *                  may be NULL)
 *   tiles        = work items {r, s, c0, nc} (4 int32 each): candidates
 *                  [c0, c0+nc) of request r, slot s, nc <= *tile_m, covering
 *                  every query row once, ordered by L_r descending (ties by
 *                  r), then candidate block, then slot.  Capacity
 *                  xattn_max_tiles() entries.
 *   n_tiles[0]   = number of tiles (device int32).
 * *tile_m (host) receives the candidates-per-tile used by xattn_forward for
 * this batch shape.  `workspace` as for xattn_forward. */
xattn_status xattn_plan(xattn_ctx* ctx,
                        const int32_t* cu_seqlens_kv, const int32_t* cu_cand,
                        int32_t num_requests, int32_t total_cand,
                        int32_t total_kv, int32_t heads,
                        int32_t* cu_q, int32_t* row_req, int32_t* tiles,
                        int32_t* n_tiles, int32_t* tile_m,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Upper bound on the number of tiles xattn_plan can emit for this shape. */
int64_t xattn_max_tiles(const xattn_ctx* ctx, int32_t num_requests,
                        int32_t total_cand, int32_t heads);

/* Number of kernel launches xattn_forward enqueues for this batch shape (for
 * callers that capture or time it): 1 on XATTN_PATH_SINGLE and
 * XATTN_PATH_SHORT, 2 on XATTN_PATH_GEMM, 3 in fp32 mode.
 * Returns 0 for invalid arguments or a batch without query rows. */
int32_t xattn_forward_launches(const xattn_ctx* ctx, int32_t num_requests,
                               int32_t total_cand, int32_t total_kv, int32_t heads);

/* Kernels xattn_forward (and xattn_attend, minus the planner) runs for this
 * batch shape. */
typedef enum {
    XATTN_PATH_SINGLE = 1,  /* attention kernel plans and projects (<= 16 requests) */
    XATTN_PATH_GEMM = 2,    /* projection GEMM with the planner, then attention      */
    XATTN_PATH_FP32 = 3,    /* fp32 planner, projection and attention kernels        */
    XATTN_PATH_SHORT = 4    /* short-memory kernel: plan, projection and attention in
                               one launch                                            */
} xattn_path;

/* The xattn_path of this batch shape, or 0 for invalid arguments or a batch
 * without query rows. */
int32_t xattn_forward_path(const xattn_ctx* ctx, int32_t num_requests,
                           int32_t total_cand, int32_t total_kv, int32_t heads);

/* TSP query projection alone (Eq. (8) applied to W_Q of Eq. (7)):
 * Q[row] = Z[row] . W_Q[row % q], Q [total_cand][q][d] in the context's
 * dtype (bf16: fp32 accumulation, rounded to nearest-even) - the same kernel
 * xattn_forward runs into its workspace. */
xattn_status xattn_project(xattn_ctx* ctx, const void* Z, const void* W_Q,
                           int32_t total_cand, void* Q, void* stream);

/* Output gate and output projection of Eq. (7) (ReST reading note, s.3.3.1),
 * the gate projection token-specific as in Eq. (8) (s.3.3.2), W_o shared by
 * all slots:
 *     Y[row] = ( O[row] * sigmoid( Z[row] . W_go[s] ) ) . W_o     (row = c*q + s)
 * with O the attention output of xattn_forward for the same batch.
 *   - Z, O, Y  [total_cand][q][d] in the context's type;
 *   - W_go     [q][d][d] output-major: W_go[s][o][i] multiplies Z[.][i] into
 *              gate feature o (like W_Q);
 *   - W_o      [d][d] output-major: W_o[p][o] multiplies gated feature o into
 *              Y[.][p].
 * Two launches on `stream`: the gate GEMM (sigmoid and product with O in its
 * epilogue; bf16: the gated values are rounded to bf16) writing the last
 * total_cand*q*d elements of `workspace` - the projected-query region of a
 * workspace sized by xattn_workspace_size, so a plan stored there is kept -
 * then the W_o GEMM.  In bf16 on a model of d = 256 with at least one unit
 * of 64 candidates x slot per compute unit it is one launch with the same
 * arithmetic (bit for bit) that keeps the gated values on chip (the
 * workspace is then not written).  `workspace_bytes` must cover that region either way.  Errors:
 * XATTN_EINVAL for NULL pointers or a negative count; XATTN_EWORKSPACE for a
 * small workspace; XATTN_EHIP for a launch failure. */
xattn_status xattn_output(xattn_ctx* ctx, const void* Z, const void* W_go, const void* O,
                          const void* W_o, int32_t total_cand, void* Y, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Synchronise `stream` and read the device-side validation flag a previous
 * xattn_forward / xattn_plan left in `workspace`: *flag = 0 when the offset
 * arrays were consistent, otherwise a bitmask (1: cu_seqlens_kv, 2: cu_cand).
 * Returns XATTN_OK when the flag is 0 and XATTN_EDEVICE_VALIDATION when it is
 * not (that call then computed nothing); XATTN_EINVAL / XATTN_EHIP when the
 * flag could not be read.  Clears nothing. */
xattn_status xattn_device_error(xattn_ctx* ctx, const void* workspace,
                                int32_t* flag, void* stream);

/* Text describing the last failure on the calling thread ("" if none).
 * Valid until the next xattn call on this thread. */
const char* xattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H */
