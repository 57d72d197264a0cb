/*
 * anchor_attn.h -- C ABI of the MI355X (gfx950) AnchorFormer anchor-attention library.
 *
 * What it computes (AnchorFormer, arXiv 2505.16463; Pith verdict page: referee report
 * summary for Eq. (11) and the Eq. (12) multiplication order, desk-editor letter for A
 * row-stochastic and Delta the diagonal of its column sums; paper abstract for the
 * anchors as neurons of a layer and the O(mn) cost):
 *
 *   for every batch b and head j, with q = Q[b,j] (n x d), v = V[b,j] (n x d) and the
 *   head's anchors u = U[j] (m x d):
 *       A     = rowsoftmax(q u^T / sqrt(d))          n x m, softmax over the m anchors
 *       Delta = diag(1^T A)                          column sums (anchor degrees)
 *       H[b,j] = A (Delta^-1 (A^T v))                n x d, never forming an n x n matrix
 *   An anchor whose column sum is exactly 0 contributes nothing (its row of
 *   Delta^-1 A^T v is taken as 0).
 *
 * Layouts: Q, V and H are [B, h, n, d] and U is [h, m, d], all contiguous row-major
 * (d fastest).  U is shared by every batch element (anchors are per-head parameters).
 * Q, U, V and H have one element type (fp32 or bf16); accumulation is fp32 and the
 * output is rounded to nearest-even.
 *
 * Memory and ownership: all four pointers are device pointers on the context's device,
 * owned by the caller, 16-byte aligned; H must not overlap Q, U or V.  The context owns
 * a grow-only device workspace used by long sequences: the first call that needs a
 * larger workspace allocates it (hipMalloc, which may synchronize); later calls of the
 * same or smaller size allocate nothing.  A workspace outgrown by a later call is kept
 * (not freed) until anchor_attn_destroy, so a graph captured before the growth still
 * replays on valid memory.  A context must not be used by two host threads at once, and
 * calls on one context that may run concurrently on different streams share that
 * workspace and race: give each stream its own context (contexts are cheap; each owns
 * only its workspaces).  Once an eager call of a shape has sized the workspaces, calls of
 * that shape allocate nothing, record no memset and can be captured into a HIP graph.
 * Test hook: when the environment variable ANCHOR_ATTN_FAIL_ALLOC_ABOVE holds a decimal
 * byte count at anchor_attn_create, that context's device allocations above it fail with
 * ANCHOR_ATTN_ERROR_OUT_OF_MEMORY (as a full device would).
 *
 * Errors: every function returns a status; nothing is thrown, printed or aborted across
 * this boundary.  All arguments are validated before any work is enqueued, so on an
 * error return nothing ran and H is untouched.  A failed launch returns
 * ANCHOR_ATTN_ERROR_HIP; faults during execution surface at the caller's next
 * synchronisation.
 */
#ifndef ANCHOR_ATTN_H
#define ANCHOR_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct anchor_attn_ctx anchor_attn_ctx;   /* opaque */

typedef enum {
    ANCHOR_ATTN_FP32 = 0,
    ANCHOR_ATTN_BF16 = 1
} anchor_attn_dtype_t;

typedef enum {
    ANCHOR_ATTN_SUCCESS = 0,
    ANCHOR_ATTN_ERROR_INVALID_VALUE = 1,   /* null pointer, negative size, m or d == 0, overlap, misalignment */
    ANCHOR_ATTN_ERROR_NOT_SUPPORTED = 2,   /* d, m or dtype outside the entry point's domain, plan not applicable */
    ANCHOR_ATTN_ERROR_OUT_OF_MEMORY = 3,   /* workspace allocation failed; the context stays usable */
    ANCHOR_ATTN_ERROR_HIP = 4              /* HIP runtime error (no device, launch failure) */
} anchor_attn_status_t;

/* Plans: how a call is mapped onto kernels.  AUTO picks per shape.  FUSED computes a
 * (batch, head) slice in one kernel without workspace (short sequences, n <= 1024,
 * m <= 64, bf16 only): one workgroup per slice, or two workgroups for a slice, each writing one half of
 * the output dims: at d = 64 for some slices when there are fewer than two slices per CU,
 * at d = 128 for every slice.  SPLIT
 * splits the tokens of a slice over workgroups: pass 1 writes per-chunk partial column
 * sums and A^T V, a finalize kernel reduces them in a fixed order into
 * Delta^-1 A^T V, and pass 2 recomputes A and writes H. */
typedef enum {
    ANCHOR_ATTN_PLAN_AUTO = 0,
    ANCHOR_ATTN_PLAN_FUSED = 1,
    ANCHOR_ATTN_PLAN_SPLIT = 2
} anchor_attn_plan_t;

/* Creates a context bound to the calling thread's current HIP device.
 * out: receives the handle (NULL -> INVALID_VALUE).  No device -> ERROR_HIP. */
anchor_attn_status_t anchor_attn_create(anchor_attn_ctx** out);

/* Releases the context and its workspace (hipFree synchronizes the device).
 * ctx == NULL is a no-op returning SUCCESS. */
anchor_attn_status_t anchor_attn_destroy(anchor_attn_ctx* ctx);

/* Enqueues H = A (Delta^-1 (A^T V)) on `stream` (a hipStream_t; NULL = default stream)
 * and returns without waiting.
 *   Q, V, H : [B, h, n, d]  device, element type `dtype`
 *   U       : [h, m, d]     device, element type `dtype`
 * Domain: B, h, n >= 0 (B*h*n == 0 is a successful no-op); 1 <= m <= 512 (more than 256
 * anchors: dtype BF16 with d <= 64, run by the split plan); d in {32, 64},
 * or d = 128 with dtype BF16 (the fused plan takes m <= 32 with n <= 256 and m <= 64 with
 * n <= 1024; PLAN_FUSED gives NOT_SUPPORTED beyond that) or with dtype FP32 and m <= 128
 * (the split plan); other d, or d = 128 in FP32 above 128 anchors, give NOT_SUPPORTED.
 * m >= n is accepted (the result is still defined; the O(mn) saving needs m < n). */
anchor_attn_status_t anchor_attn_forward(anchor_attn_ctx* ctx,
                                         const void* Q, const void* U, const void* V, void* H,
                                         int B, int h, int n, int m, int d,
                                         anchor_attn_dtype_t dtype, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): anchor_attn_forward with the split
 * plan's partials in a fixed scratch array of 64 MiB in device memory that the library
 * holds on every GPU it runs on until the process ends, instead of the context's
 * workspace.  It calls no allocating routine; the context only supplies its device, CU
 * count and plan setting.  Arguments, layouts, domain and errors as anchor_attn_forward
 * (contiguous tensors), plus: a shape whose split-plan partials exceed 64 MiB returns
 * ANCHOR_ATTN_ERROR_NOT_SUPPORTED with nothing enqueued (32 slices of 16384 tokens with
 * 256 anchors at d = 64 need ~35 MiB).  All calls on one GPU share its scratch, which
 * keeps the last call's contents (every call writes each partial before reading it, so
 * nothing needs clearing): calls that may overlap on one GPU (other streams, other
 * threads, other contexts) race and must be serialised by the caller. */
anchor_attn_status_t anchor_attn_forward_noalloc(anchor_attn_ctx* ctx,
                                                 const void* Q, const void* U, const void* V,
                                                 void* H, int B, int h, int n, int m, int d,
                                                 anchor_attn_dtype_t dtype, void* stream);

/* The same forward on strided views, so that Q and V can be read where a fused projection
 * left them (for example the two halves of a packed [B, n, 2, h, d] or [B, n, 3, h, d]
 * tensor) and H written straight into a [B, n, h, d] layout for the output projection
 * (the block around the attention: Pith verdict page, supporting citations of the DeiT /
 * LeViT backbones the layer is dropped into).
 *   q_strides, v_strides, h_strides: host arrays of three element strides (batch, head,
 *     token) of the [B, h, n, d] views of Q, V and H; the d values of a token are
 *     contiguous.  NULL means the contiguous layout (h*n*d, n*d, d).
 * Each stride must be >= 0 and a multiple of 16 bytes, and the base pointers 16-byte
 * aligned; distinct rows of H must not share an element, and H's span (first to last
 * element) must not overlap the spans of Q, V or U.  Otherwise INVALID_VALUE.  Inputs may
 * alias each other.  Everything else as anchor_attn_forward, which is this call with
 * three NULL stride arrays. */
anchor_attn_status_t anchor_attn_forward_strided(anchor_attn_ctx* ctx,
                                                 const void* Q, const long long* q_strides,
                                                 const void* U,
                                                 const void* V, const long long* v_strides,
                                                 void* H, const long long* h_strides,
                                                 int B, int h, int n, int m, int d,
                                                 anchor_attn_dtype_t dtype, void* stream);

/* The attention block around the layer, the way a ViT block's self-attention is replaced
 * by it (Pith verdict page: AnchorFormer as a drop-in attention module in DeiT / LeViT
 * backbones; the pages print no projections, so this is the plain reading): for tokens
 * X [B, n, C] with C = h*d,
 *   [Q | V] = X Wqv + bqv       Wqv [C, 2C], bqv [2C]; head j owns columns j*d .. j*d+d-1
 *                               of Q and C + j*d .. of V (no key projection: the anchors
 *                               U take the keys' place)
 *   H       = anchor attention of every (batch, head) slice with U [h, m, d]
 *   Y       = H Wo + bo         H [B, n, C] with head-major columns, Wo [C, C], bo [C]
 * All row-major bf16 device arrays; fp32 accumulation; Q, V and H are rounded to bf16
 * between the steps.  bqv and bo may be NULL (no bias).  With d <= 64, m <= 32 and n <= 256
 * (a ViT-S/16 block, say) and any plan but PLAN_SPLIT, one kernel per (batch, head) slice
 * projects that slice's Q and V from X on the matrix cores and runs the attention on them
 * (no Q|V tensor in memory); otherwise the Q|V projection runs through hipBLASLt and the
 * attention through the kernels of anchor_attn_forward_strided reading the projection in
 * place.  The output projection runs through hipBLASLt.  The context keeps a second
 * workspace for the projection, H and hipBLASLt (grown on demand; growth synchronizes).  The first call of a new shape also
 * times hipBLASLt's candidate algorithms on the call's own operands and synchronizes the
 * stream; later calls of that shape only enqueue.  Y must not overlap any input.
 * Domain: dtype BF16 (else NOT_SUPPORTED); B, n, h >= 0 (no tokens: a no-op); m and d as
 * anchor_attn_forward.  Argument errors: nothing is enqueued; a HIP error in a later step
 * can leave the earlier steps enqueued. */
anchor_attn_status_t anchor_attn_block_forward(anchor_attn_ctx* ctx,
                                               const void* X, const void* Wqv, const void* bqv,
                                               const void* U, const void* Wo, const void* bo,
                                               void* Y, int B, int n, int h, int m, int d,
                                               anchor_attn_dtype_t dtype, void* stream);

/* A second O(n) attention from the pages, sharing the reduce-then-apply structure: the
 * ReLU kernel linear attention of the L2ViT page (Eq. (4): the decomposable kernel
 * identity with phi = ReLU, the denominator clamped below at Cmin = 1e2 there), per
 * (batch, head) slice of Q, K, V, O [B, h, n, d] (strided views as in
 * anchor_attn_forward_strided; NULL strides = contiguous):
 *   out_i = phi(qscale * q_i) (phi(K)^T V) / max(phi(qscale * q_i) . (phi(K)^T 1), cmin)
 * qscale stands for 1/s, the page's learnable scale; since phi(a q) = a phi(q) it only
 * moves the clamp.  bf16 in and out, fp32 accumulation (phi(K)^T V rounded to bf16 as a
 * matrix-core operand).  With enough slices one workgroup per slice (Q, K, V read once,
 * O written once; at d = 128 two workgroups per slice, one per half of the output dims,
 * each reading all of Q and K); with fewer than half a slice per CU, or under PLAN_SPLIT,
 * the tokens of a slice are split over workgroups (partial sums in the context's workspace,
 * reduced in a fixed order).
 * Domain: dtype BF16 (else NOT_SUPPORTED), d in {32, 64, 128}, B, h, n >= 0 (no tokens: a
 * no-op), cmin > 0 and qscale > 0 finite (else INVALID_VALUE); views as for
 * anchor_attn_forward_strided (O's rows distinct, O's span disjoint from the inputs').
 * Errors: nothing is enqueued. */
anchor_attn_status_t anchor_attn_relu_linear_forward(anchor_attn_ctx* ctx,
                                                     const void* Q, const long long* q_strides,
                                                     const void* K, const long long* k_strides,
                                                     const void* V, const long long* v_strides,
                                                     void* O, const long long* o_strides,
                                                     int B, int h, int n, int d, float cmin,
                                                     float qscale, anchor_attn_dtype_t dtype,
                                                     void* stream);

/* Nystrom attention with given landmark tokens (Fast Nystrom Attention page, key
 * machinery): the attention matrix approximated by three row softmaxes through s landmark
 * rows q = Q[idx], k = K[idx], the middle one inverted.  Per (batch b, head j) slice of
 * Q, K, V, H [B, h, n, d] (contiguous, row-major), with c = 1/sqrt(d):
 *   F1 = rowsoftmax(Q k^T c) (n x s),  F2 = rowsoftmax(q k^T c) (s x s),
 *   F3 = rowsoftmax(q K^T c) (s x n),  H = F1 (F2^-1 (F3 V)),
 * never forming an n x n matrix.  idx: device int32 [B, s], the landmark token indices of
 * each batch element (shared by its heads; the page picks them by farthest-point
 * sampling, which is the caller's business here).  Indices are expected distinct and in
 * [0, n); out-of-range values are clamped to that range.  Repeated indices make F2
 * singular and the output non-finite.  bf16 in and out, fp32 accumulation; F2 in fp32
 * and its solve in fp64 (Gauss-Jordan with partial pivoting: F2's condition number reaches
 * 1e14 when a sink token is among the landmarks), F1, F3 and Z = F2^-1 F3 V rounded to
 * bf16 as matrix-core operands.  Uses the context's workspace (grown on demand;
 * growth synchronizes).
 * Domain: dtype BF16 (else NOT_SUPPORTED), d in {32, 64} with 1 <= s <= 128, or d = 128
 * with 1 <= s <= 96 (else NOT_SUPPORTED), s <= n (else INVALID_VALUE); B, h, n >= 0 with no tokens a no-op.  All
 * pointers 16-byte aligned (idx 4-byte); H must not overlap Q, K, V or idx.
 * Errors: nothing is enqueued. */
anchor_attn_status_t anchor_attn_nystrom_forward(anchor_attn_ctx* ctx, const void* Q,
                                                 const void* K, const void* V, const int* idx,
                                                 void* H, int B, int h, int n, int s, int d,
                                                 anchor_attn_dtype_t dtype, void* stream);

/* Enqueues the gradients of anchor_attn_forward for a loss L with dL/dH = dH (AnchorFormer
 * abstract: the anchors are learnable, so the layer is trained through; the Pith verdict
 * page's Eq. (11) in the Eq. (12) order is the function differentiated), on `stream`,
 * without waiting:
 *   Q, V, dH, dQ, dV : [B, h, n, d]  device, bf16 or fp32 (dtype)
 *   U, dU            : [h, m, d]     device, same dtype; dU is summed over the batch (U is
 *                                    shared by every batch element)
 * Accumulation is fp32; bf16 results are rounded from it.  The fp32 path keeps every
 * operand in fp32 (full fp32 matrix-core products) and holds the n x m_pad matrix dS in
 * the workspace (4 bytes per element).  dQ, dU and dV are written in full
 * (dU is zero when B*h*n == 0); they must not overlap each other or any input.  The
 * context's workspace grows as for the split plan (the first call of a larger shape may
 * synchronize).  Domain: as anchor_attn_forward, with dtype BF16 and either d in {32, 64}
 * with m <= 256 or d = 128 with m <= 128, or dtype FP32 with d in {32, 64} and m <= 256 or
 * d = 128 and m <= 128 (split plan only: a context whose plan is FUSED returns
 * NOT_SUPPORTED for fp32); larger m returns NOT_SUPPORTED.
 * Errors as anchor_attn_forward: nothing is enqueued and no output is touched. */
anchor_attn_status_t anchor_attn_backward(anchor_attn_ctx* ctx,
                                          const void* Q, const void* U, const void* V,
                                          const void* dH, void* dQ, void* dU, void* dV,
                                          int B, int h, int n, int m, int d,
                                          anchor_attn_dtype_t dtype, void* stream);

/* The backward on strided views (as anchor_attn_forward_strided: host arrays of three
 * element strides (batch, head, token), NULL = contiguous) for Q, V, dH and the outputs
 * dQ, dV; U and dU stay contiguous [h, m, d].  dQ's and dV's rows must be distinct and the
 * outputs' spans must not overlap each other or any input's span.  Everything else as
 * anchor_attn_backward, which is this call with five NULL stride arrays. */
anchor_attn_status_t anchor_attn_backward_strided(anchor_attn_ctx* ctx,
                                                  const void* Q, const long long* q_strides,
                                                  const void* U,
                                                  const void* V, const long long* v_strides,
                                                  const void* dH, const long long* dh_strides,
                                                  void* dQ, const long long* dq_strides,
                                                  void* dU,
                                                  void* dV, const long long* dv_strides,
                                                  int B, int h, int n, int m, int d,
                                                  anchor_attn_dtype_t dtype, void* stream);

/* Forces a plan for later forward calls on this context (tests and tuning); AUTO
 * restores the default choice.  A forced plan that cannot run a given shape makes that
 * forward call return NOT_SUPPORTED. */
anchor_attn_status_t anchor_attn_set_plan(anchor_attn_ctx* ctx, anchor_attn_plan_t plan);

/* Writes a one-line, NUL-terminated description of the plan a forward call with these
 * arguments would use (kernels, grids, chunking, workspace bytes) into buf[0..len).
 * Validates like anchor_attn_forward but enqueues nothing and allocates nothing. */
anchor_attn_status_t anchor_attn_describe_plan(anchor_attn_ctx* ctx, int B, int h, int n,
                                               int m, int d, anchor_attn_dtype_t dtype,
                                               char* buf, int len);

/* Static, human-readable name of a status code (never NULL). */
const char* anchor_attn_status_string(anchor_attn_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* ANCHOR_ATTN_H */
