/*
 * usaf.h -- C ABI of the MI355X (gfx950) sparse MoE fine-tuning hot path.
 *
 * The method is USAF as described on the author's GitHub page
 * ("tsuyu122/usaf" README): native fine-tuning of about 0.5% of the real
 * expert weights of a Mixture-of-Experts layer, chosen by gradient magnitude
 * ("how it works": importance bullet), with the router trained densely
 * ("how it works": router bullet), the active set re-chosen by RigL every 50
 * steps ("how it works": sparsity bullet), SparseAdam as the optimiser (A100
 * per-operation table) and 4-bit experts dequantised once into resident
 * copies ("how it works": caching bullet; quantisation recipe).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers   device pointers unless marked HOST.
 * Ownership  the caller owns every buffer.  The library never allocates
 *            device memory; scratch comes from a caller workspace whose
 *            size usaf_workspace_size() reports.
 * Streams    every call only enqueues work on `stream` (0 = the null stream)
 *            and returns without synchronising, except where noted.
 * Errors     every call returns a usaf_status; nothing is printed, nothing
 *            throws, no environment variable is read.  Arguments are
 *            validated before anything is enqueued: on an error return no
 *            work was enqueued and no output was touched.  A shape the
 *            kernels do not handle is refused with USAF_ERR_UNSUPPORTED,
 *            never served by a slower fallback.
 * Layouts    row-major throughout.  One layer's expert weights live in one
 *            flat buffer Wflat of N = 3*E*H*I elements:
 *              [ gate_up (E, 2I, H) | down (E, H, I) ]
 *            (the fused expert tensors of the README's quantisation recipe,
 *            stored out x in); rows [0, I) of gate_up[e] are the gate
 *            projection, rows [I, 2I) the up projection.  A flat index is a
 *            plain offset into Wflat.  The router Wr is a separate fp32 [E, H].
 * Dtypes     `act` selects the activation / expert-weight type: USAF_F32
 *            (float) or USAF_BF16 (bf16 stored as uint16).  Router weights,
 *            routing weights, gradients of weights and Adam moments are fp32.
 *            Accumulation is fp32.
 * Determinism every output is bit-identical across repeated calls with the
 *            same inputs (no floating-point atomics).
 */
#ifndef USAF_H
#define USAF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define USAF_API __attribute__((visibility("default")))
#else
#define USAF_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  USAF_OK = 0,
  USAF_ERR_INVALID_ARG = 1,   /* null required pointer, bad size, K > E, k > N, ... */
  USAF_ERR_UNSUPPORTED = 2,   /* a shape or dtype the kernels refuse                 */
  USAF_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required          */
  USAF_ERR_HIP = 4,           /* a HIP launch or copy failed                         */
  USAF_ERR_NOT_IMPLEMENTED = 5
} usaf_status;

typedef enum { USAF_F32 = 0, USAF_BF16 = 1 } usaf_dtype;

/* Which call a workspace is sized for (usaf_workspace_size). */
typedef enum {
  USAF_WS_FORWARD = 0,
  USAF_WS_BACKWARD = 1,
  USAF_WS_TOPK = 2,
  USAF_WS_RIGL = 3,
  USAF_WS_MASKED_PLAN = 4,
  USAF_WS_UNION = 5
} usaf_ws_kind;

/* One MoE layer: T tokens, hidden H, E experts, top-K routing, expert
 * intermediate size I, activation dtype act (a usaf_dtype).  S = T*K slots.
 * Supported: T >= 1, 1 <= K <= E <= 1024, H % 64 == 0, I % 32 == 0,
 * 3*E*H*I < 2^32, T*K < 2^31. */
typedef struct {
  int32_t T, H, E, K, I;
  int32_t act;
} usaf_moe_shape;

/* Per-layer state written by the forward (and the backward) and read by the
 * backward.  All buffers are caller-owned device memory.  "Expert-major"
 * rows are ordered by expert, and by slot id within an expert: row p holds
 * slot perm[p].  A slot is s = t*K + j (token t, j-th chosen expert). */
typedef struct {
  float   *logits;    /* [T, E]   fp32 router logits (forward writes)              */
  int32_t *topk_ids;  /* [T, K]   chosen experts, logit descending, ties lowest id  */
  float   *topk_w;    /* [T, K]   routing weights: softmax over the K chosen logits */
  int32_t *offsets;   /* [E + 1]  expert-major start row of each expert; [E] = S    */
  int32_t *perm;      /* [S]      slot id at each expert-major row                  */
  int32_t *slot_pos;  /* [S]      expert-major row of each slot (inverse of perm)   */
  void    *gu;        /* [S, 2I]  act: pre-activation [gate | up], expert-major     */
  void    *a;         /* [S, I]   act: silu(gate) * up, expert-major                */
  void    *dgu;       /* [S, 2I]  act: d[gate | up] (backward writes)               */
  float   *dw;        /* [T, K]   fp32 d loss / d routing weight (backward writes)  */
} usaf_moe_state;

/* Statistics of one RigL reselection (device memory, written by the call). */
typedef struct {
  int64_t n_drop;           /* entries dropped from the active set (= r)            */
  int64_t n_grow;           /* entries grown into it (= r)                          */
  int64_t topk_new_vs_old;  /* |TopK_k(|g|) \ S_old|: entries of a fresh top-k that */
                            /* are not in the old set (the README's "turnover")     */
} usaf_rigl_stats;

/* Bytes of workspace `kind` needs for `shape` (FORWARD, BACKWARD,
 * MASKED_PLAN: the plan of usaf_masked_plan for any list) or for a
 * selection over n keys picking k (TOPK: n = N, k; RIGL: n = N, k = active
 * count) or for usaf_sorted_union of lists totalling n entries (UNION).
 * `shape` may be NULL for TOPK / RIGL / UNION.  Result goes to HOST *bytes.
 * Returns USAF_ERR_INVALID_ARG for a bad kind, size or null `bytes`. */
USAF_API usaf_status usaf_workspace_size(int32_t kind, const usaf_moe_shape *shape, int64_t n,
                                int64_t k, size_t *bytes /* HOST */);

/* MoE layer forward (README "how it works": tokens are routed to a handful of
 * experts; the router is the gating network trained alongside).
 *   logits = X * Wr'^T  (Wr' = bf16(Wr) for bf16 layers, Wr for fp32 layers)
 *   per token: the K largest logits (ties: lowest expert id), routing weights
 *   = softmax over those K logits; slots grouped by expert (stable); per
 *   expert SwiGLU: [g|u] = x W_gu^T, a = silu(g)*u, y = a W_d^T;
 *   Y[t] = sum_{j=0..K-1} w[t,j] * y[t*K+j]   (fixed j order).
 * X [T,H] act; Wr [E,H] fp32; Wflat [N] act; Y [T,H] act (written);
 * state: logits, topk_ids, topk_w, offsets, perm, slot_pos, gu, a written.
 * ws: USAF_WS_FORWARD bytes. */
USAF_API usaf_status usaf_moe_forward(const usaf_moe_shape *shape, const void *X, const float *Wr,
                             const void *Wflat, void *Y, const usaf_moe_state *state,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* Expert weights of one layer in the pages' own 4-bit storage (README "how
 * it works": experts kept in 4-bit HQQ form; quantisation recipe: groups
 * along the input dimension), the affine codes of usaf_dequant_affine:
 *   gate_up: q_gu [E*2I, H/2] bytes, s_gu and z_gu [E*2I, H/group] fp16 bits
 *   down:    q_d  [E*H,  I/2] bytes, s_d  and z_d  [E*H,  I/group] fp16 bits
 * w = bf16(fp32(fp32(q - z) * s)), element 2i in the low nibble of byte i;
 * rows in the flat order of the resident weights. */
typedef struct {
  const uint8_t *q_gu; const uint16_t *s_gu; const uint16_t *z_gu;
  const uint8_t *q_d;  const uint16_t *s_d;  const uint16_t *z_d;
  int32_t group;  /* 64 or 128; for usaf_moe_forward_q4, 2 * group must divide H and I */
} usaf_q4_experts;

/* The layer forward of usaf_moe_forward with the expert weights read from
 * their 4-bit codes and dequantised as the GEMMs load them, no resident
 * copy (README "how it works": caching bullet -- the pages keep resident
 * dequantised copies; this is the other side of that trade, for layers that
 * only run forward, such as the frozen lower layers of a partly trained
 * stack).  Every output and every field of `state` it writes equals, bit for
 * bit, usaf_moe_forward on the usaf_dequant_affine copy of the same codes.
 * bf16 layers only (UNSUPPORTED otherwise); the code arrays must be 16-byte
 * aligned and the scale and zero arrays 4-byte aligned (UNSUPPORTED
 * otherwise).  ws: USAF_WS_FORWARD bytes. */
USAF_API usaf_status usaf_moe_forward_q4(const usaf_moe_shape *shape, const void *X, const float *Wr,
                                         const usaf_q4_experts *w, void *Y,
                                         const usaf_moe_state *state, void *ws, size_t ws_bytes,
                                         hipStream_t stream);

/* Plan of the masked gradient for one active list idx[nnz] (strictly
 * ascending): where every (expert, row, column tile) segment starts in the
 * list, and the list's work cut into tiles of balanced entry counts.  It
 * depends on idx and the shape only (not on routing or data), so a caller
 * that keeps the list for many steps builds it once per list (README "how it
 * works": the active set changes only at RigL reselection) and passes it to
 * usaf_masked_backward.  plan: device buffer of usaf_workspace_size
 * (USAF_WS_MASKED_PLAN) bytes, written; its layout is private to the library.
 * fp32 layers need no plan (returns OK, writes nothing).  Errors:
 * INVALID_ARG for nnz < 0, nnz > N or idx == NULL with nnz > 0; WORKSPACE
 * for a short buffer. */
USAF_API usaf_status usaf_masked_plan(const usaf_moe_shape *shape, const uint32_t *idx, int64_t nnz,
                             void *plan, size_t plan_bytes, hipStream_t stream);

/* Masked backward (README intro and A100 table: gradients only for the
 * selected subset of expert weights; the router gradient is dense).
 * Reads the forward's state and dY [T,H] (act).  Writes
 *   state->dgu, state->dw;
 *   dWr [E,H] fp32: dense router gradient (straight-through the bf16 cast);
 *   dX [T,H] act (nullable: skipped when NULL);
 *   dW: for a sparse list idx[nnz] (strictly ascending flat indices) dW[i] is
 *       the fp32 gradient at idx[i]; in dense mode (idx == NULL and
 *       nnz == N) dW[f] is the gradient of every expert weight f.
 * plan (nullable): usaf_masked_plan's plan of this very idx[nnz]; with NULL
 * the plan is rebuilt inside ws on every call.  Ignored in dense mode.  The
 * plan records the list it was built for (nnz, the idx address, the first and
 * last entry); when these differ from the call's list the gradient kernels
 * write no dW value and raise *nonfinite (when given), so that a step
 * using a stale plan is skipped rather than computed from another list's
 * tiles.  A list rewritten in place with the same length and end entries is
 * not detected: rebuild the plan whenever the list changes.
 * nonfinite (nullable, device int32): incremented when any dW value or dWr
 * is NaN/Inf (sparse mode); the caller zeroes it before the step.
 * An empty list (nnz == 0, idx may be NULL) computes everything but dW.
 * ws: USAF_WS_BACKWARD bytes.  Errors: INVALID_ARG for nnz < 0, nnz > N, a
 * null required pointer, or idx == NULL with 0 < nnz < N; UNSUPPORTED for a
 * sparse list on a bf16 layer whose X (T*H*2 bytes) or expert-major dgu
 * (T*K*2I*2 bytes) reaches 4 GiB, or with T*K >= 2^24. */
USAF_API usaf_status usaf_masked_backward(const usaf_moe_shape *shape, const void *X, const float *Wr,
                                 const void *Wflat, const usaf_moe_state *state,
                                 const void *dY, const uint32_t *idx, int64_t nnz,
                                 const void *plan, float *dW, float *dWr, void *dX,
                                 int32_t *nonfinite, void *ws, size_t ws_bytes, hipStream_t stream);

/* Importance selection (README "how it works": the 0.5% of weights with the
 * largest gradient magnitude).  Ranks grad[0..n) by (|grad| descending, index
 * ascending), |grad| compared as fp32 bit patterns (NaN ranks above +Inf),
 * and writes the first k indices to out_idx [k] in ascending order.
 * exclude (nullable) is a strictly ascending list of n_exclude indices that
 * may not be chosen (RigL grow).  out_val (nullable) receives grad at
 * out_idx.  grad and ws must be 16-byte aligned (UNSUPPORTED otherwise).
 * Errors: INVALID_ARG when k > n - n_exclude, n >= 2^32 or n_exclude > n.
 * ws: USAF_WS_TOPK bytes for n (about 16n bytes: the candidates' keys and
 * indices are buffered). */
USAF_API usaf_status usaf_importance_topk(const float *grad, int64_t n, int64_t k,
                                 const uint32_t *exclude, int64_t n_exclude,
                                 uint32_t *out_idx, float *out_val,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

/* RigL reselection (README "how it works": sparsity bullet, RESELECT_EVERY).
 *   D = the r entries of old_idx with the smallest |Wflat| (ties: lowest index)
 *   G = the r entries outside old_idx with the largest |grad| (ties: lowest)
 *   new_idx = sort((old_idx \ D) u G)                       [k], ascending
 *   new_m, new_v: moments of kept entries carried over, zero for grown ones.
 * Weights are not modified.  grad [N] fp32 (a dense scan's dW); Wflat [N]
 * (shape->act); old_w (nullable, shape->act, [k]): Wflat at old_idx, e.g.
 * usaf_sparse_adam's compact list, read in order instead of gathering the
 * drop keys from Wflat; old_idx [k] strictly ascending; old_m, old_v [k] fp32.
 * new_w (nullable, shape->act, [k]; needs old_w): Wflat at new_idx, the kept
 * entries' weights copied from old_w and the grown ones' read from Wflat
 * (the new compact list of usaf_sparse_adam, without a gather of the list).
 * stats (nullable, device): counts, including the fresh top-k's novelty.
 * Outputs must not alias inputs; grad and ws 16-byte aligned (UNSUPPORTED
 * otherwise).  Errors: INVALID_ARG for r > k, k > N, r > N - k, new_w
 * without old_w.
 * ws: USAF_WS_RIGL bytes for (N, k). */
USAF_API usaf_status usaf_rigl_reselect(const usaf_moe_shape *shape, const float *grad,
                               const void *Wflat, const void *old_w, const uint32_t *old_idx,
                               const float *old_m, const float *old_v, int64_t k, int64_t r,
                               uint32_t *new_idx, float *new_m, float *new_v, void *new_w,
                               usaf_rigl_stats *stats, void *ws, size_t ws_bytes,
                               hipStream_t stream);

/* SparseAdam (README A100 table) -- Adam, Kingma & Ba 2015 Algorithm 1, on
 * a list of entries:  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 * w -= lr * (m / (1-b1^step)) / (sqrt(v / (1-b2^step)) + eps).
 * W (w_dtype: USAF_BF16 updated with one round-to-nearest-even, or USAF_F32)
 * is updated in place at idx[i] (idx NULL = dense: entry i is W[i]); g, m, v
 * are [n] fp32 aligned with idx; m, v are updated in place.  step >= 1 is the
 * step number after incrementing.  The hyper-parameters are taken in double:
 * 1-beta and the bias corrections 1-beta^step are formed in double on the
 * host and rounded once to fp32 (a float beta2 = 0.999f would shift 1-beta2
 * by 1.3e-5 relative).  skip_if_nonzero (nullable, device int32):
 * when it holds a non-zero value the kernel changes nothing (the NaN-step
 * skip of the README's results table); the caller then does not advance its
 * step counter.  idx entries must be distinct.
 * w_list (nullable, w_dtype, [n]): a compact copy of W[idx[i]].  When given
 * (idx must be too) the weights are read from w_list[i] instead of the
 * scattered W[idx[i]] and written to both, so the list stays equal to W at
 * idx; build it with usaf_gather and rebuild it after the list changes.
 * Errors: INVALID_ARG for n < 0, step < 1, null W/g/m/v, w_list without idx. */
USAF_API usaf_status usaf_sparse_adam(int32_t w_dtype, void *W, const uint32_t *idx, int64_t n,
                             void *w_list, const float *g, float *m, float *v, int64_t step,
                             double lr, double beta1, double beta2, double eps,
                             const int32_t *skip_if_nonzero, hipStream_t stream);

/* out[i] = W[idx[i]] for i < n (w_dtype elements): the compact weight list
 * of usaf_sparse_adam.  Errors: INVALID_ARG for n < 0 or null pointers with
 * n > 0, or an unknown w_dtype. */
USAF_API usaf_status usaf_gather(int32_t w_dtype, const void *W, const uint32_t *idx, int64_t n,
                        void *out, hipStream_t stream);

/* W[idx[i]] = vals[i] for i < n (w_dtype elements): a compact list written
 * back into the flat weights, the inverse of usaf_gather (README "how it
 * works": only the selected subset is trained, so a checkpoint holds the
 * trained weights as such a list).  Also the plain scattered write that
 * usaf_sparse_adam's own write-back of the list is measured against.  The
 * idx entries must be distinct (which of two equal entries' values lands is
 * unspecified).  Errors: INVALID_ARG for n < 0 or null pointers with n > 0,
 * or an unknown w_dtype. */
USAF_API usaf_status usaf_scatter(int32_t w_dtype, void *W, const uint32_t *idx, int64_t n,
                         const void *vals, hipStream_t stream);



/* Resident dequantisation (README "how it works": caching bullet; dequant
 * once, keep the working copy).  Symmetric int4: q [rows, cols/2] bytes,
 * element 2i in the low nibble of byte i, two's complement in [-8, 7];
 * scale_f16 [rows, cols/group] fp16 bit patterns; out_bf16 [rows, cols]
 * bf16 = round_to_nearest_even(q * scale) (the product is exact, so this is
 * the only rounding).  Supported: group == 64, cols % 64 == 0.
 * Errors: INVALID_ARG for rows < 0 or null pointers; UNSUPPORTED otherwise. */
USAF_API usaf_status usaf_dequant_resident(const uint8_t *q, const uint16_t *scale_f16, int64_t rows,
                                  int64_t cols, int32_t group, void *out_bf16,
                                  hipStream_t stream);

/* The pages' own 4-bit storage (README "how it works": experts read in 4-bit
 * HQQ format; its quantisation recipe quantises with group size 128),
 * dequantised once into resident bf16.  Affine codes: q [rows, cols/2]
 * bytes, element 2i in the low nibble of byte i, unsigned in [0, 15];
 * scale_f16 and zero_f16 [rows, cols/group] fp16 bit patterns; out_bf16
 * [rows, cols] = round_to_nearest_even_bf16(fp32(fp32(q - zero) * scale)):
 * the difference and the product are each rounded once in fp32.
 * Supported: group 64 or 128, cols % group == 0, q 4-byte and out 16-byte
 * aligned.  Errors: INVALID_ARG for rows or cols < 0 or null pointers with a
 * non-empty shape; UNSUPPORTED otherwise. */
USAF_API usaf_status usaf_dequant_affine(const uint8_t *q, const uint16_t *scale_f16,
                                const uint16_t *zero_f16, int64_t rows, int64_t cols,
                                int32_t group, void *out_bf16, hipStream_t stream);

/* ---- helpers of the step (not method steps of their own) -------------- */

/* Regression loss of a layer output: loss = mean((Y - tgt)^2) over T*H
 * elements (fp32, device scalar), dY = 2 (Y - tgt) / (T*H) in act dtype.
 * nonfinite (nullable) is incremented when the loss is NaN/Inf.
 * ws: 4 * ceil(T*H / 4096) + 64 bytes at least (usaf_workspace_size FORWARD
 * is always enough). */
USAF_API usaf_status usaf_mse_grad(const usaf_moe_shape *shape, const void *Y, const void *tgt,
                          void *dY, float *loss, int32_t *nonfinite, void *ws,
                          size_t ws_bytes, hipStream_t stream);

/* The loss above without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * usaf_mse_grad, bit for bit; its partial sums live in a fixed 256 KiB
 * device array of the library instead of a workspace, one copy per device,
 * held until the process ends.  Limit: T*H <= 2^28 elements, else
 * USAF_ERR_UNSUPPORTED.  Nothing carries over between calls, but every call
 * on one device uses the same array: calls that overlap on one device (on
 * different streams, or from different threads) race.  The stream must
 * belong to the current device.  USAF_ERR_HIP if the array's device address
 * cannot be obtained. */
USAF_API usaf_status usaf_mse_grad_noalloc(const usaf_moe_shape *shape, const void *Y,
                                           const void *tgt, void *dY, float *loss,
                                           int32_t *nonfinite, hipStream_t stream);

/* Residual stream of a stack of layers (the stacked-layer workload's
 * composition reading: no attention or norm between the MoE layers, so the
 * next layer's input is the sum of a layer's input and output, and in the
 * backward the gradient of a layer's input is the sum of the gradient of
 * the next layer's input and the layer's own dX): out[i] = round_act(a[i] +
 * b[i]) for i < n, act USAF_BF16 (round to nearest even) or USAF_F32.  a, b,
 * out: device arrays of n elements; out may alias a or b.  Asynchronous on
 * `stream`.  Errors: INVALID_ARG for n < 0, an unknown act, or null pointers
 * with n > 0. */
USAF_API usaf_status usaf_residual_add(int32_t act, const void *a, const void *b, void *out,
                              int64_t n, hipStream_t stream);

/* Sorted union of two strictly ascending u32 lists a[na] and b[nb] (the
 * bookkeeping of a training run that keeps every index ever selected, since
 * RigL keeps the trained values of the entries it drops: README "how it
 * works", sparsity bullet).  out (capacity na + nb, must not alias a or b)
 * receives the union, strictly ascending, and *n_out (device int64) its
 * length.  ws: USAF_WS_UNION bytes for n = na + nb.  Errors: INVALID_ARG for
 * negative sizes, na + nb >= 2^32 or null pointers where entries exist;
 * WORKSPACE for a short ws. */
USAF_API usaf_status usaf_sorted_union(const uint32_t *a, int64_t na, const uint32_t *b, int64_t nb,
                                       uint32_t *out, int64_t *n_out, void *ws, size_t ws_bytes,
                                       hipStream_t stream);

/* out[i] = in[i + 1] - in[i] for i < n (int32): the slots each expert
 * received from the forward's offsets (the router load-balance monitor of a
 * training run).  Errors: INVALID_ARG for n < 0 or null pointers with n > 0. */
USAF_API usaf_status usaf_adjacent_diff(const int32_t *in, int64_t n, int32_t *out,
                                        hipStream_t stream);

/* Routing alone, from given fp32 logits [T, E]: writes state->topk_ids,
 * topk_w, offsets, perm, slot_pos exactly as usaf_moe_forward does. */
USAF_API usaf_status usaf_route(const usaf_moe_shape *shape, const float *logits,
                       const usaf_moe_state *state, hipStream_t stream);

/* ---- measurement hook ----------------------------------------------------
 * Kernel classes that can be timed.  While one class is armed, every launch
 * of that class (a GEMM, or the whole kernel sequence of a selection)
 * records a HIP event before and after itself on its own stream; up to
 * `capacity` launches are recorded.  For benchmarking only: the hook is
 * process-global and not thread-safe.  The events are created by
 * usaf_timer_arm (no device memory is allocated) and read back with
 * usaf_timer_read, which waits for them. */
typedef enum {
  USAF_K_ROUTER_GEMM = 0, USAF_K_ROUTE = 1, USAF_K_GATE_UP = 2, USAF_K_DOWN = 3,
  USAF_K_COMBINE_Y = 4, USAF_K_DA = 5, USAF_K_ROUTER_BWD = 6, USAF_K_DX = 7,
  USAF_K_COMBINE_DX = 8, USAF_K_MASKED_DW = 9, USAF_K_DENSE_DW = 10, USAF_K_MSE = 11,
  USAF_K_ADAM = 12, USAF_K_DEQUANT = 13, USAF_K_TOPK = 14, USAF_K_RIGL_MERGE = 15,
  USAF_K_COUNT = 16
} usaf_kernel_class;

/* Arm class `kernel_class` (-1 disarms) for up to `capacity` (1..65536)
 * launches; resets the count.  Errors: INVALID_ARG, HIP (event creation). */
USAF_API usaf_status usaf_timer_arm(int32_t kernel_class, int32_t capacity);

/* Wait for the recorded events and write the milliseconds of each recorded
 * launch to HOST ms[0..count), count <= capacity. */
USAF_API usaf_status usaf_timer_read(float *ms /* HOST */, int32_t capacity,
                                     int32_t *count /* HOST */);

/* Human-readable name of a status code (static string). */
USAF_API const char *usaf_status_string(usaf_status s);

/* Library version, as major*10000 + minor*100 + patch. */
USAF_API int32_t usaf_version(void);

#ifdef __cplusplus
}
#endif
#endif /* USAF_H */
