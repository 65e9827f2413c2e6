/*
 * attn.h - C ABI of the causal softmax attention library for MI355X (gfx950).
 *
 * The operation (pages: "Show HN: automatic deduction of FlashAttention kernel
 * from 25 lines of SQL", neshdevtech.com, the view `attention` in its window
 * and GROUP BY spellings, the GRADIENT statement and the NADARAYA_WATSON
 * query):
 *
 *   s_ij = scale * sum_d q_id k_jd          for every pair j <= i (j > i: absent)
 *   o_i  = sum_{j<=i} softmax_j(s_i.) v_j    an absent pair contributes nothing,
 *                                            so an infinity in v_j reaches only
 *                                            rows i >= j
 *   lse_i = ln sum_{j<=i} exp(s_ij)          natural log of the scaled scores
 *
 * and the gradient of a loss L whose upstream gradient is dout = dL/do
 * (for the pages' loss sum(o^2)/2, dout = o).
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, contiguous, row-major [B, H, N, D] (q, k, v, o, dout,
 *     dq, dk, dv) or [B, H, N] (lse).  Each (b, h) is one independent head.
 *   - Every pointer is device memory owned by the caller, 16-byte aligned (4-byte
 *     for the float columns of nw_gauss_average).  The library never
 *     allocates, frees or synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream).
 *     ATTN_OK means every launch was accepted; results are valid once the
 *     caller has synchronised the stream.  A device fault surfaces there.
 *   - Errors: a non-zero return; no launch has been made for ATTN_EINVAL and
 *     ATTN_EUNSUPPORTED.  attn_last_error() returns the calling thread's last
 *     message.  The library keeps no other state; calls from several host
 *     threads are safe.
 *   - Outputs must not alias inputs, except dout == o in the backward passes.
 *   - Size limits of the attention entry points (ATTN_EINVAL beyond them):
 *     N <= 2^24, B*H <= 2^24, and (B*H rounded up to a multiple of 8) *
 *     ceil(N / 32) < 2^24, so that no launch exceeds 2^32 work-items.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, o, dout, dq, dk, dv.  Arithmetic: ATTN_F64 in
 * float64 throughout; ATTN_F32 in float32; ATTN_BF16 multiplies bfloat16
 * operands with float32 accumulation and float32 softmax.  lse is float64 for
 * ATTN_F64 and float32 otherwise. */
typedef enum { ATTN_F64 = 0, ATTN_F32 = 1, ATTN_BF16 = 2 } attn_dtype_t;

enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,       /* null pointer, size < 1, bad scale/denominator, short workspace */
  ATTN_EUNSUPPORTED = 2, /* a valid request this build does not implement (D != 64) */
  ATTN_EHIP = 3          /* the HIP runtime rejected a launch */
};

/* Join predicate: which (query i, key j) pairs exist (pages: "Show HN:
 * automatic deduction of FlashAttention kernel from 25 lines of SQL", the view
 * `attention` joins q and k on q.t >= k.t, and the same post's claim that the
 * fused plan follows for any softmax-weighted join).  An absent pair takes no
 * part in the max, the sum or the weighted average.
 *   ATTN_MASK_CAUSAL  j <= i                          (the view `attention`)
 *   ATTN_MASK_FULL    every j                          (the join with no predicate)
 *   ATTN_MASK_WINDOW  j <= i and i - j < window        (a causal band of `window`
 *                     keys; window >= 1, and a window >= N is the causal mask) */
typedef enum { ATTN_MASK_CAUSAL = 0, ATTN_MASK_FULL = 1, ATTN_MASK_WINDOW = 2 } attn_mask_t;

/* Forward pass (the view `attention`: scores from the join q.t >= k.t, the
 * row max subtracted, normalised by the row sum, weighted sum of v).
 *   dtype  attn_dtype_t of q, k, v, o
 *   B, H   batch and heads, >= 1;  N tokens per head, >= 1;  D features, must be 64
 *   scale  multiplier of q.k, finite and > 0 (the pages use 1/8 = 1/sqrt(64))
 *   q, k, v  inputs [B, H, N, D];  o output [B, H, N, D];  lse output [B, H, N]
 * Returns ATTN_OK / ATTN_EINVAL / ATTN_EUNSUPPORTED / ATTN_EHIP. */
ATTN_API int attn_causal_fwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                    const void* q, const void* k, const void* v, void* o, void* lse,
                    void* stream);

/* The forward pass under any join predicate of attn_mask_t: as
 * attn_causal_fwd, with
 *   mask    ATTN_MASK_CAUSAL, ATTN_MASK_FULL or ATTN_MASK_WINDOW
 *   window  keys per query for ATTN_MASK_WINDOW (>= 1); ignored otherwise
 * attn_causal_fwd(...) is attn_fwd(..., ATTN_MASK_CAUSAL, 0, ...).
 * Returns ATTN_OK / ATTN_EINVAL (also for an unknown mask or window < 1) /
 * ATTN_EUNSUPPORTED / ATTN_EHIP. */
ATTN_API int attn_fwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                      attn_mask_t mask, int64_t window, const void* q, const void* k, const void* v,
                      void* o, void* lse, void* stream);

/* Bytes of device workspace attn_causal_bwd needs for these sizes.  On a
 * request attn_causal_bwd would reject (bad dtype or sizes) it returns 0 and
 * sets attn_last_error(); a caller that then passes a 0-byte workspace gets
 * ATTN_EINVAL from attn_causal_bwd, before any launch.  The caller allocates
 * the workspace; its contents need not be initialised and are garbage
 * afterwards. */
ATTN_API size_t attn_causal_bwd_workspace_bytes(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D);

/* Backward pass: dq, dk, dv of a loss with upstream gradient dout (the pages'
 * GRADIENT statement: grad(loss, q.x), grad(loss, k.x), grad(loss, v.x) of
 * loss = SUM(x * x) / 2, computed in one backward pass; pass dout = o for it).
 * Scores are recomputed from q, k and the saved lse of attn_causal_fwd (same
 * dtype, sizes and scale).
 *   o, dout   [B, H, N, D] (may be the same pointer);  lse [B, H, N]
 *   dq, dk, dv  outputs [B, H, N, D] in dtype
 *   workspace   device memory of at least attn_causal_bwd_workspace_bytes()
 * Returns ATTN_OK / ATTN_EINVAL / ATTN_EUNSUPPORTED / ATTN_EHIP. */
ATTN_API int attn_causal_bwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                    const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const void* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * attn_causal_bwd with the same arguments minus the workspace.  Its
 * workspace is a static device array of ATTN_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; the call
 * itself allocates nothing.
 *   - Sizes whose workspace (attn_causal_bwd_workspace_bytes) exceeds
 *     ATTN_NOALLOC_SCRATCH_BYTES are refused with ATTN_EINVAL before any
 *     launch: up to 2,096,896 rows (B*H*N) for bfloat16 and float64
 *     (8 bytes of workspace per row), 4,193,792 for float32 (4 bytes).
 *   - All calls on one GPU share that GPU's array: two calls whose work can
 *     overlap on one GPU (different streams, or different host threads) race
 *     and give wrong gradients.  Calls on one stream are ordered and safe.
 *   - The array of the device current at the call is used; the stream must
 *     belong to that device.  Nothing in the array needs clearing between
 *     calls (the backward writes every value before reading it).
 * Returns ATTN_OK / ATTN_EINVAL / ATTN_EUNSUPPORTED / ATTN_EHIP. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
ATTN_API int attn_causal_bwd_noalloc(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D,
                                     double scale, const void* q, const void* k, const void* v,
                                     const void* o, const void* dout, const void* lse, void* dq,
                                     void* dk, void* dv, void* stream);

/* Workspace bytes for attn_bwd (the same for every mask; equal to
 * attn_causal_bwd_workspace_bytes). */
ATTN_API size_t attn_bwd_workspace_bytes(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D);

/* The backward pass under any join predicate: as attn_causal_bwd, with mask
 * and window as in attn_fwd; lse must come from attn_fwd with the same mask
 * and window.  attn_causal_bwd(...) is attn_bwd(..., ATTN_MASK_CAUSAL, 0, ...).
 * Returns ATTN_OK / ATTN_EINVAL (also for an unknown mask or window < 1) /
 * ATTN_EUNSUPPORTED / ATTN_EHIP. */
ATTN_API int attn_bwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                      attn_mask_t mask, int64_t window, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const void* lse, void* dq, void* dk,
                      void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Segment predicate: attn_fwd / attn_bwd with one more condition on the
 * join, equality of a per-token segment id (pages: "Show HN: automatic
 * deduction of FlashAttention kernel from 25 lines of SQL", the demo script's
 * claim that its fusion rule covers any softmax-weighted join, and its check
 * that masks are rows absent from the join).  The pair (i, j) exists when
 * mask / window admit it AND seg[b][i] == seg[b][j]; so documents packed
 * into one sequence attend only within themselves.
 *   seg   device int32 [B, N], 4-byte aligned, shared by the H heads of each
 *         batch; any values (equal ids need not be contiguous).  Read only;
 *         no output or workspace may overlap it.
 *   lse for attn_bwd_seg must come from attn_fwd_seg with the same seg, mask
 *   and window.  Every row keeps at least the pair (i, i), so no row is empty.
 * Other arguments, workspace size included, as attn_fwd / attn_bwd.
 * Returns ATTN_OK / ATTN_EINVAL (also for a null seg) / ATTN_EUNSUPPORTED /
 * ATTN_EHIP. */
ATTN_API int attn_fwd_seg(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D,
                          double scale, attn_mask_t mask, int64_t window, const int32_t* seg,
                          const void* q, const void* k, const void* v, void* o, void* lse,
                          void* stream);
ATTN_API int attn_bwd_seg(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D,
                          double scale, attn_mask_t mask, int64_t window, const int32_t* seg,
                          const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const void* lse, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Training step of the pages' GRADIENT statement (loss = SUM(x * x) / 2 over
 * every output value, so the upstream gradient is dout = o), with the loss
 * fused into the forward:
 * attn_fwd_train is attn_fwd that also
 *   - writes *loss = sum(o^2) / 2 (one float64 in device memory, summed in a
 *     fixed order from the stored o, so repeated calls give the same bits), and
 *   - fills `workspace` (at least attn_bwd_workspace_bytes()) with the per-row
 *     values the backward of that loss needs;
 * attn_bwd_from_fwd is then attn_bwd(..., dout = o, ...) reading those values
 * instead of recomputing them (one kernel fewer).  Pass it the same sizes,
 * scale, mask, window, q, k, v, o, lse and workspace, unchanged in between.
 * Returns ATTN_OK / ATTN_EINVAL / ATTN_EUNSUPPORTED / ATTN_EHIP. */
ATTN_API int attn_fwd_train(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                            attn_mask_t mask, int64_t window, const void* q, const void* k,
                            const void* v, void* o, void* lse, void* workspace,
                            size_t workspace_bytes, double* loss, void* stream);
ATTN_API int attn_bwd_from_fwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                               attn_mask_t mask, int64_t window, const void* q, const void* k,
                               const void* v, const void* o, const void* lse, void* dq, void* dk,
                               void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Nadaraya-Watson control (the pages' NADARAYA_WATSON query): for every target
 * p, out_p = sum_q w_pq v_q / sum_q w_pq over ALL sources q (a cross join),
 * w_pq = exp(-((tx_p - sx_q)^2 + (ty_p - sy_q)^2) / denom).  The pages use
 * denom = 0.25.  float32 columns (struct of arrays), float32 arithmetic with
 * a per-target running max subtracted before exp.
 *   n_targets, n_sources >= 1;  denom finite and > 0
 * Returns ATTN_OK / ATTN_EINVAL / ATTN_EHIP. */
ATTN_API int nw_gauss_average(int64_t n_targets, const float* tx, const float* ty, int64_t n_sources,
                     const float* sx, const float* sy, const float* sv, float denom,
                     float* out, void* stream);

/* ---- Steps before the path ------------------------------------------------
 *
 * The long table <-> matrix adapter (pages: "Show HN: automatic deduction of
 * FlashAttention kernel from 25 lines of SQL", the demo script's helpers
 * table() and matrix()).  The SQL engines hold a T x D matrix as the long
 * table (t, d, x): one row per cell, t and d its row and column positions.
 * Columns are separate arrays: t[rows], d[rows] (int64) and x[rows] (the
 * element type `dtype`).  The matrix is dense row-major [T, D] of `dtype`.
 *
 * attn_matrix_to_table: the T*D rows of matrix m in (t, d) order (row
 *   r = t*D + d), the order of the forward's ORDER BY t, d.  Values are copied
 *   bit for bit.  All four pointers 16-byte aligned.  The outputs must not
 *   overlap each other or m.
 *
 * attn_table_to_matrix: the pivot.  Cell (t, d) of m receives the x of the row
 *   naming it, bit for bit; a cell no row names is a quiet NaN.  A row whose
 *   coordinate lies outside [0, T) x [0, D) is skipped, and a cell named by
 *   two rows is an error: the call writes to the device word *status 0 when
 *   neither happened, else the OR of 1 (some coordinate out of range) and 2
 *   (some cell named twice), in which case m is unspecified.  The caller reads
 *   *status after synchronising the stream.  `workspace` holds
 *   attn_table_workspace_bytes(dtype, T, D) bytes of scratch: 256 bytes, then
 *   one staging word per cell (4 bytes for ATTN_BF16, 8 for ATTN_F32, 16 for
 *   ATTN_F64), then for tables of at least 65536 cells about 4 MiB more (the
 *   counts of a sort of the rows by cell block); it needs no initialisation.
 *   The call makes no per-row device atomic: a doubly named cell is found by
 *   counting.
 *   Alignment: t, d 8 bytes; x one element; m and workspace 16 bytes;
 *   status 4 bytes.  m, the workspace and status must not overlap the inputs
 *   or each other.  At most 2^40 rows and 2^40 cells (ATTN_EINVAL).
 *   attn_table_workspace_bytes returns 0 (and sets attn_last_error()) for a
 *   dtype or sizes the call would reject. */
ATTN_API int attn_matrix_to_table(attn_dtype_t dtype, int64_t T, int64_t D, const void* m, int64_t* t,
                                  int64_t* d, void* x, void* stream);
ATTN_API size_t attn_table_workspace_bytes(attn_dtype_t dtype, int64_t T, int64_t D);
ATTN_API int attn_table_to_matrix(attn_dtype_t dtype, int64_t rows, const int64_t* t, const int64_t* d,
                                  const void* x, int64_t T, int64_t D, void* m, int32_t* status,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* The query, key and value input projections (pages: the "Wiki notes" page,
 * brainpick-2k7.pages.dev, its MLIR functions @attention_head and
 * @mini_attention: Q = x Wq, K = x Wk, V = x Wv).  x is [B, N, Dm] (one
 * embedding row per token); each weight is [Dm, H*64] with head h in columns
 * 64h .. 64h+63 (no bias, no scale).  q, k, v are written as the attention
 * takes them, [B, H, N, 64]:  q[b][h][n][j] = sum_c x[b][n][c] wq[c][64h + j].
 * One launch forms all three from one read of x.  Arithmetic: float64 for
 * ATTN_F64, float32 for ATTN_F32; ATTN_BF16 multiplies bfloat16 operands
 * with float32 accumulation and rounds the results to bfloat16 (nearest even).
 * All pointers 16-byte aligned; the outputs must not overlap each other or
 * the inputs.  Limits (ATTN_EINVAL): sizes >= 1, H <= 65535, B*N < 2^31,
 * N <= 2^24, x and each weight at most 2^40 elements. */
ATTN_API int attn_qkv_project(attn_dtype_t dtype, int64_t B, int64_t N, int64_t Dm, int64_t H,
                              const void* x, const void* wq, const void* wk, const void* wv,
                              void* q, void* k, void* v, void* stream);

/* Profiling hook: timing events around one kernel.  Kernels are named by
 * slot: ATTN_TIMER_FWD (the forward kernel), ATTN_TIMER_BWD_PRE (the
 * backward's per-row delta kernel), ATTN_TIMER_BWD_DKDV (dK/dV), ATTN_TIMER_BWD_DQ
 * (dQ), ATTN_TIMER_NW (the Nadaraya-Watson kernel), ATTN_TIMER_TABLE (the
 * pivot's scatter kernel of attn_table_to_matrix), ATTN_TIMER_PROJECT (the
 * kernel of attn_qkv_project).  While a slot is set (per
 * host thread), each call that launches that kernel records `start` on its
 * stream just before the launch and `stop` just after it, so hipEventElapsedTime
 * gives the kernel's duration.  Both are hipEvent_t created by the caller; pass
 * NULL, NULL to clear the slot.  Returns ATTN_OK, or ATTN_EINVAL for an unknown
 * slot or when exactly one event is NULL. */
enum {
  ATTN_TIMER_FWD = 0,
  ATTN_TIMER_BWD_PRE = 1,
  ATTN_TIMER_BWD_DKDV = 2,
  ATTN_TIMER_BWD_DQ = 3,
  ATTN_TIMER_NW = 4,
  ATTN_TIMER_TABLE = 5,
  ATTN_TIMER_PROJECT = 6,
  ATTN_TIMER_SLOTS = 7
};
ATTN_API int attn_set_kernel_timer(int slot, void* start, void* stop);

/* Message of the calling thread's most recent error ("" if none).  The pointer
 * stays valid until that thread's next call into the library.  This mirrors
 * how the demo script of "Show HN: automatic deduction of FlashAttention
 * kernel from 25 lines of SQL" treats a failing engine (its report.attempt
 * helper records the failure and the run goes on): every entry point returns
 * a code instead of aborting, and the message says what failed. */
ATTN_API const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
