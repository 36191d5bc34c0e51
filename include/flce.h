/*
 * flce.h -- C ABI of the MI355X (gfx950) fused linear cross-entropy library.
 *
 * Fused linear cross-entropy (FLCE) is the lm_head projection of hidden states
 * onto the vocabulary fused with the cross-entropy loss and its backward pass,
 * so that the [tokens, vocab] logits tensor is never materialised:
 *   - Liger-Kernel commit e6a81bb0c3 ("Muse Glimmer" support), Summary item 1
 *     (fused linear + cross-entropy / skip-logits path), Summary item 2 (token
 *     accuracy), Details > Softcap (T * tanh(logits * m / T), with the output
 *     multiplier m folded onto the hidden-state side), Memory (fp32
 *     [vocab, hidden] weight-gradient accumulator);
 *   - Liger-Kernel commit 40a9d8a61b ("DeepSeek-V3" support), Summary (logits
 *     never materialised in training with labels) and Memory (chunked
 *     transients plus a fixed fp32 weight-gradient accumulator).
 *
 * Per call, for N tokens with hidden size H and vocabulary V:
 *   a     = m * (h W^T)                          [N, V], never stored whole
 *   z     = T * tanh(a / T)     (T > 0), else a
 *   lse_i = log sum_v exp(z_iv)
 *   loss  = s * sum_{valid i} (lse_i - z_{i, label_i}),
 *           s = 1 / N_valid (mean; 0 if N_valid = 0) or 1 (sum)
 *   pred_i = lowest v with z_iv = max_v z_iv;  n_correct = #{valid i : pred_i = label_i}
 *   G_iv  = s * (softmax(z_i)_v - [v = label_i]) * (1 - (z_iv / T)^2)  on valid rows, 0 otherwise
 *   grad_h = m * G W        [N, H], dtype of h
 *   grad_W = m * G^T h      [V, H], fp32 (overwritten, not accumulated)
 * A row is valid when label_i != ignore_index.  flce_fwd_bwd takes the
 * upstream gradient of the scalar loss as 1; flce_fwd_bwd_ex adds an upstream
 * gradient, per-row outputs, per-row losses without reduction and
 * accumulation into grad_W (flce_options_t), and flce_fwd computes the loss
 * alone.
 *
 * The library allocates no device memory and never synchronises inside
 * flce_fwd_bwd, flce_fwd_bwd_ex or flce_fwd: all work is enqueued on the
 * caller's stream and the caller owns every buffer, including the workspace.
 */
#ifndef FLCE_H_
#define FLCE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype of h, W and grad_h. */
typedef enum { FLCE_DTYPE_BF16 = 0, FLCE_DTYPE_F32 = 1 } flce_dtype;

/*
 * Reduction of the per-row losses.  FLCE_REDUCTION_NONE (flce_fwd_bwd_ex and
 * flce_fwd only) keeps the per-row losses (options.loss_rows, required): the
 * scalar `loss` then receives their sum and row i's gradient is scaled by the
 * upstream gradient options.grad_rows[i] (1 when grad_rows is NULL).
 */
typedef enum { FLCE_REDUCTION_MEAN = 0, FLCE_REDUCTION_SUM = 1, FLCE_REDUCTION_NONE = 2 } flce_reduction;

/* Return codes. */
enum {
  FLCE_OK = 0,
  FLCE_EINVAL = 1,        /* bad argument: null pointer, bad size, bad enum, misalignment */
  FLCE_EWORKSPACE = 2,    /* workspace smaller than flce_workspace_size() for the call */
  FLCE_EDEVICE = 3,       /* a HIP launch or runtime call failed */
  FLCE_ELABEL = 4,        /* (device-detected) a label outside [0, V) that is not ignore_index */
  FLCE_EUNSUPPORTED = 5,  /* valid but unsupported shape, e.g. H not a multiple of 8 (bf16) / 4 (fp32) or too large */
  FLCE_ESCRATCH = 6       /* flce_fwd_bwd_noalloc: no chunk plan fits its static scratch (FLCE_NOALLOC_SCRATCH_BYTES) */
};

/*
 * Chunk plan.  Tokens are processed in chunks of `chunk_rows` rows; one chunk's
 * logits (padded to `vocab_padded` columns) is the largest transient, so the
 * full [N, V] logits never exist ("chunked transients", DeepSeek-V3 page,
 * Memory).  chunk_rows <= ceil(N / 2), hence at least two chunks for N >= 2.
 */
typedef struct {
  int64_t chunk_rows;         /* C: tokens per chunk */
  int64_t n_chunks;           /* ceil(N / C) (0 when N = 0) */
  int64_t vocab_padded;       /* V rounded up to the 256-column tile */
  int64_t split_k;            /* grad_h = G W is split over the vocabulary into this many parts */
  size_t logits_chunk_bytes;  /* C * vocab_padded * sizeof(dtype) */
  size_t workspace_bytes;     /* total workspace this plan needs */
  size_t grad_W_bytes;        /* 4 * V * H: the caller's fp32 weight-gradient accumulator */
} flce_plan_t;

/*
 * Compute the chunk plan for a call with these sizes that may use at most
 * `budget_bytes` of workspace (0 = default budget: 16 GiB for the chunk
 * transients plus the packed copy of the valid rows of h).  Pure host
 * arithmetic; no GPU needed.  Returns FLCE_OK, FLCE_EINVAL (negative sizes,
 * bad dtype, null `out`), FLCE_EUNSUPPORTED (H not a multiple of 8 for bf16 or
 * 4 for fp32; H > 2^21; V above 2^22 - 256 for bf16 or 2^21 - 256 for fp32;
 * N >= 2^31) or FLCE_EWORKSPACE (not even the smallest chunk fits).
 */
int flce_plan(int64_t N, int64_t H, int64_t V, int dtype, size_t budget_bytes, flce_plan_t* out);

/*
 * Workspace bytes needed by flce_fwd_bwd for these sizes under `budget_bytes`
 * (0 = default budget).  Returns 0 if no plan exists (see flce_plan).  Passing
 * exactly this many bytes to flce_fwd_bwd reproduces the same plan.
 */
size_t flce_workspace_size(int64_t N, int64_t H, int64_t V, int dtype, size_t budget_bytes);

/*
 * Forward and backward of fused linear cross-entropy (see the top of this
 * file for the formulas and sources).
 *
 * Arguments (all pointers are device pointers unless stated):
 *   h          [N, H] row-major, dtype; 16-byte aligned.  Read only.
 *   W          [V, H] row-major (nn.Linear weight layout), dtype; 16-byte aligned.  Read only.
 *   labels     [N] int64; 8-byte aligned.  Read only.
 *   N, H, V    N >= 0, H >= 1, V >= 1; H % 8 == 0 (bf16) or H % 4 == 0 (fp32).
 *   ignore_index  rows with this label are excluded from the loss, from
 *              n_correct and from the gradients.
 *   softcap_T  logit softcap T; T <= 0 disables the cap.  Finite; with a cap,
 *              1 / T and m / T must be finite as well.
 *   multiplier output multiplier m, applied to the logits before the cap; finite.
 *   reduction  FLCE_REDUCTION_MEAN or FLCE_REDUCTION_SUM (NONE: flce_fwd_bwd_ex).
 *   loss       [1] fp32, written.
 *   grad_h     [N, H] dtype, written (gradient w.r.t. the caller's h); 16-byte aligned.
 *   grad_W     [V, H] fp32, overwritten with this call's gradient; 16-byte aligned.
 *   n_correct  [1] int64, written with the count of valid rows whose argmax is
 *              the label; may be NULL.
 *   stream     HIP stream on which every kernel is enqueued (0 = null stream).
 *   dtype      FLCE_DTYPE_BF16 or FLCE_DTYPE_F32.
 *   workspace  device scratch owned by the caller, 256-byte aligned, at least
 *              flce_workspace_size(N, H, V, dtype, 0) bytes (or the size for the
 *              budget the caller planned with).  Its contents on entry are
 *              ignored; on return it holds the status word read by
 *              flce_read_status.
 *   workspace_bytes  size of `workspace`; the chunk plan is the largest that fits.
 *
 * Errors: argument checks run on the host before anything is enqueued; on
 * FLCE_EINVAL / FLCE_EUNSUPPORTED / FLCE_EWORKSPACE no output is touched.
 * FLCE_EDEVICE means a launch failed (outputs unspecified).  Labels outside
 * [0, V) that are not ignore_index are detected on the device: outputs are
 * then unspecified and flce_read_status returns FLCE_ELABEL.
 * N = 0 or no valid row gives loss = 0, n_correct = 0 and zero gradients.
 * Calls on distinct workspaces may run concurrently; two calls sharing a
 * workspace must be ordered (same stream).
 *
 * Ignored rows add nothing to the loss or to either gradient, so the call
 * first packs the valid rows of h (in order) into the workspace and runs the
 * GEMMs over those alone; the chunks then cover packed rows.  The results are
 * those of the definition above; only the rounding order of grad_W's sum
 * over tokens and of the loss sum depends on which rows are packed together.
 * (flce_fwd_bwd_ex and flce_fwd skip the packing when every row's
 * log-sum-exp or argmax is requested: those are defined for ignored rows too.)
 */
int flce_fwd_bwd(const void* h, const void* W, const int64_t* labels,
                 int64_t N, int64_t H, int64_t V,
                 int64_t ignore_index, float softcap_T, float multiplier, int reduction,
                 float* loss, void* grad_h, float* grad_W, int64_t* n_correct,
                 hipStream_t stream, int dtype, void* workspace, size_t workspace_bytes);

/*
 * Options of flce_fwd_bwd_ex and flce_fwd.  The per-row outputs and the
 * upstream gradient complete the output contract of the Liger-Kernel pages
 * (Muse Glimmer page, Testing Done: the token_accuracy / predicted_tokens
 * contract; DeepSeek-V3 page, Summary: token_accuracy / predicted_tokens
 * returned); accumulation into grad_W serves gradient accumulation over
 * micro-batches (SpecForge page, Changes: accumulation prepass).
 * Zero-initialise the struct and set what is needed: every NULL output is
 * skipped and, with use_grad_scale = 0, the upstream gradient is 1.  All
 * pointers are device pointers.
 */
typedef struct {
  float* loss_rows;        /* [N] fp32 out: lse_i - z_{i,label_i} on valid rows, 0 on ignored
                              rows; 4-byte aligned; required with FLCE_REDUCTION_NONE */
  float* lse_rows;         /* [N] fp32 out: log-sum-exp of every row's capped logits */
  int64_t* pred_rows;      /* [N] int64 out: first argmax of every row's capped logits
                              (the predicted token); 8-byte aligned */
  const float* grad_rows;  /* [N] fp32 in: upstream gradient of each row's loss; only with
                              FLCE_REDUCTION_NONE (NULL = 1 for every row) */
  float grad_scale;        /* upstream gradient of the scalar loss, used when use_grad_scale
                              is 1: multiplies grad_h and this call's grad_W term (0 gives a
                              zero grad_h and a zero grad_W term); finite */
  int accumulate_grad_W;   /* 0: grad_W = this call's gradient; 1: grad_W += it (grad_W must
                              hold the running sum on entry) */
  int use_grad_scale;      /* 0: grad_scale is ignored (upstream gradient 1); 1: it is used */
} flce_options_t;

/*
 * flce_fwd_bwd with options (may be NULL: then identical to flce_fwd_bwd).
 * Same arguments, workspace and errors as flce_fwd_bwd; `reduction` may also
 * be FLCE_REDUCTION_NONE.  FLCE_EINVAL also for: REDUCTION_NONE without
 * loss_rows, grad_rows with another reduction, use_grad_scale or
 * accumulate_grad_W other than 0 or 1, a non-finite grad_scale in use or a
 * misaligned row pointer.
 */
int flce_fwd_bwd_ex(const void* h, const void* W, const int64_t* labels,
                    int64_t N, int64_t H, int64_t V,
                    int64_t ignore_index, float softcap_T, float multiplier, int reduction,
                    float* loss, void* grad_h, float* grad_W, int64_t* n_correct,
                    hipStream_t stream, int dtype, void* workspace, size_t workspace_bytes,
                    const flce_options_t* options);

/*
 * flce_fwd_bwd_ex for callers that cannot allocate device memory: code under
 * HIP graph (stream) capture, tight training or serving loops, harnesses that
 * forbid allocation.  Same arguments, formulas, options and errors as
 * flce_fwd_bwd_ex except:
 *   - no workspace argument: the scratch is a static device array of
 *     FLCE_NOALLOC_SCRATCH_BYTES that each GPU running the library holds from
 *     the first call there until the process ends; the chunk plan is the
 *     largest that fits it (flce_plan with that budget), and sizes for which
 *     none fits return FLCE_ESCRATCH before anything is enqueued;
 *   - status  [1] int32 device pointer (4-byte aligned) or NULL: receives, in
 *     the call's last kernel, FLCE_OK or FLCE_ELABEL (the device-side label
 *     check that flce_read_status reports for the other entry points).
 * Nothing is allocated (no hipMalloc, no library allocation) and nothing
 * synchronises.  All calls on one GPU share its scratch and each call
 * overwrites it, so calls that overlap in time on the same GPU (different
 * streams without ordering, or different threads) race and give wrong
 * results: order them.  The first call on each device looks up the scratch's
 * device address (hipGetSymbolAddress) with that device current; the call
 * uses the current device, which must be the device of `stream`.
 */
#define FLCE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int flce_fwd_bwd_noalloc(const void* h, const void* W, const int64_t* labels,
                         int64_t N, int64_t H, int64_t V,
                         int64_t ignore_index, float softcap_T, float multiplier, int reduction,
                         float* loss, void* grad_h, float* grad_W, int64_t* n_correct, int* status,
                         hipStream_t stream, int dtype, const flce_options_t* options);

/*
 * Workspace bytes needed by flce_fwd (forward only: no logits transient and
 * no grad_h partials) under `budget_bytes` (0 = default).  0 if no plan fits
 * or the shape is unsupported.
 */
size_t flce_fwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype, size_t budget_bytes);

/*
 * Forward only: loss, n_correct and the per-row outputs of `options`, with no
 * gradient (the cross-entropy-only pass of the SpecForge page, Changes:
 * compute only the backbone CE during the accumulation prepass).  No logits
 * are stored at all, so tokens run in chunks as large as the workspace
 * allows.  Arguments as flce_fwd_bwd without grad_h and grad_W; in `options`
 * only loss_rows, lse_rows and pred_rows are used (grad_rows, grad_scale and
 * accumulate_grad_W are ignored); `workspace` holds at least
 * flce_fwd_workspace_size(N, H, V, dtype, 0) bytes.  The loss, lse and
 * argmax of each row are bitwise the ones flce_fwd_bwd computes.
 */
int flce_fwd(const void* h, const void* W, const int64_t* labels,
             int64_t N, int64_t H, int64_t V,
             int64_t ignore_index, float softcap_T, float multiplier, int reduction,
             float* loss, int64_t* n_correct,
             hipStream_t stream, int dtype, void* workspace, size_t workspace_bytes,
             const flce_options_t* options);

/*
 * Materialised-logits path: the non-fused branch the fused loss is compared
 * against (Muse Glimmer page, Testing Done: the non-fused softcap branch, and
 * skip_logits=False in evaluation; DeepSeek-V3 page, Summary: outside training
 * with labels the logits are materialised and the plain loss runs on them).
 *
 * flce_logits writes z = T tanh(m h W^T / T) (T > 0) or m h W^T, [N, V], into
 * `logits` (dtype of h; row stride `ld_logits` elements, ld_logits >= V and
 * ld_logits * sizeof(dtype) a multiple of 16; 16-byte aligned).  Columns
 * [V, ld_logits) are not written.  h, W, N, H, V, dtype as for flce_fwd_bwd.
 * Returns FLCE_OK, FLCE_EINVAL, FLCE_EUNSUPPORTED or FLCE_EDEVICE; allocates
 * nothing and needs no workspace.
 */
int flce_logits(const void* h, const void* W, int64_t N, int64_t H, int64_t V,
                float softcap_T, float multiplier, void* logits, int64_t ld_logits,
                hipStream_t stream, int dtype);

/* Workspace bytes of flce_cross_entropy for N rows (256 + 3 * N * 4, padded). */
size_t flce_cross_entropy_workspace_size(int64_t N);

/*
 * Cross-entropy of given logits z [N, V] (dtype; row stride ld_logits as for
 * flce_logits; the logits are used as they are, so a softcap belongs in
 * them): loss = s * sum_{valid i} (lse_i - z_{i,label_i}) with the reductions,
 * options and per-row outputs of flce_fwd_bwd_ex, and n_correct.  If
 * `grad_logits` is not NULL it receives d loss / d z = w_i (softmax(z_i) -
 * onehot) (w_i: reduction scale x grad_scale x grad_rows[i]; 0 on ignored
 * rows) in dtype, row stride `ld_grad` (same rules; the columns from V up to
 * the next multiple of 16 bytes are set to 0, the rest of the row is not
 * written); it may be `logits` itself (then ld_grad must equal ld_logits).
 * `workspace`: 256-byte aligned, at least flce_cross_entropy_workspace_size(N)
 * bytes; flce_read_status reports FLCE_ELABEL for out-of-range labels.
 */
int flce_cross_entropy(const void* logits, int64_t ld_logits, const int64_t* labels,
                       int64_t N, int64_t V, int64_t ignore_index, int reduction,
                       float* loss, int64_t* n_correct, void* grad_logits, int64_t ld_grad,
                       hipStream_t stream, int dtype, void* workspace, size_t workspace_bytes,
                       const flce_options_t* options);

/*
 * Upstream-gradient scaling for a training loop whose backward pass runs after
 * the fused call (DeepSeek-V3 page, Summary: in training with labels the
 * fused loss is the forward, and autograd's backward hands in the upstream
 * gradient of the loss only afterwards).  With g the fp32 value at
 * `grad_scale` (a device pointer, so the host never reads it):
 *   grad_h_out[i] = grad_h_in[i] * g   for i < n_h, both in h_dtype, computed
 *                                       in fp32 and rounded once;
 *   grad_W_out[i] = grad_W_in[i] * g   for i < n_W, read as fp32 (the fused
 *                                       call's accumulator), written in
 *                                       w_dtype (the weight's dtype).
 * Each output may be its input itself (in place; for grad_W only when w_dtype
 * is fp32) and must not otherwise overlap it.  In place with g == 1 the
 * grad_h pass writes nothing.  The h pointers may be NULL with n_h = 0, the W
 * pointers with n_W = 0.  Pointers 16-byte aligned (grad_scale 4-byte).
 * Enqueued on `stream`; no synchronisation, nothing allocated.  Returns
 * FLCE_OK, FLCE_EINVAL (null or misaligned pointer, negative size, bad dtype,
 * partly overlapping buffers) or FLCE_EDEVICE.
 */
int flce_scale_grads(const float* grad_scale, const void* grad_h_in, void* grad_h_out, int64_t n_h, int h_dtype,
                     const float* grad_W_in, void* grad_W_out, int64_t n_W, int w_dtype, hipStream_t stream);

/*
 * Synchronise `stream` and return the device-side status of the last
 * flce_fwd_bwd, flce_fwd_bwd_ex, flce_fwd or flce_cross_entropy that used
 * `workspace`: FLCE_OK or FLCE_ELABEL.  Returns
 * FLCE_EINVAL for a null workspace and FLCE_EDEVICE if the copy fails.
 */
int flce_read_status(const void* workspace, hipStream_t stream);

/*
 * After a call, a workspace also holds N_valid, the call's number of rows
 * whose label is not ignore_index, as a uint64 at byte offset
 * FLCE_WS_N_VALID_OFFSET (device memory, written on the call's stream, valid
 * until the next call that uses the workspace).  Token accuracy (Muse Glimmer
 * page, Summary item 2) is n_correct / N_valid.  The status word read by
 * flce_read_status is the int32 at byte 0.
 */
#define FLCE_WS_N_VALID_OFFSET 8

/* Static, human-readable text for a return code. */
const char* flce_strerror(int code);

/*
 * Measurement facility (not part of the method): per-kernel timing with HIP
 * events.  While enabled, every kernel that the entry points enqueue is
 * bracketed by two events recorded on the same stream, so the elapsed time is
 * that kernel's own duration on that stream.  Kinds index the arrays below.
 */
enum {
  FLCE_KERNEL_LABEL_SCAN = 0,   /* header init + label scan (N_valid, range check) and valid-row packing */
  FLCE_KERNEL_FWD_LOGITS = 1,   /* logits GEMM + softcap / LSE / argmax / label-logit epilogue */
  FLCE_KERNEL_ROW_MERGE = 2,    /* per-token log-sum-exp, loss, argmax */
  FLCE_KERNEL_GRAD_LOGITS = 3,  /* softmax - onehot (x softcap derivative), in place */
  FLCE_KERNEL_GRAD_H = 4,       /* grad_h GEMM G W (vocabulary-split partials) */
  FLCE_KERNEL_GRAD_H_REDUCE = 5,/* sum of the partials, cast to the storage dtype */
  FLCE_KERNEL_GRAD_W = 6,       /* grad_W GEMM G^T h, fp32 (overwrite, or on top of the stored grad_W) */
  FLCE_KERNEL_FINALIZE = 7,     /* loss scalar and n_correct */
  FLCE_KERNEL_ZERO = 8,         /* zero grad_W when N = 0 */
  FLCE_KERNEL_LOGITS = 9,       /* flce_logits: logits GEMM + softcap into the caller's buffer */
  FLCE_KERNEL_CROSS_ENTROPY = 10,/* flce_cross_entropy: per-row statistics (+ logit gradient) */
  FLCE_KERNEL_SCALE = 11,       /* flce_scale_grads: upstream-gradient scaling of grad_h / grad_W */
  FLCE_KERNEL_KINDS = 12
};

/* Turn event timing on (on != 0) or off for subsequent calls.  Returns FLCE_OK. */
int flce_profile_enable(int on);

/*
 * Synchronise `stream`, fold all pending event pairs into the running totals
 * and copy them out: total_ms[k] and launches[k] for k < FLCE_KERNEL_KINDS
 * (caller-owned host arrays).  reset != 0 clears the totals afterwards.
 * Returns FLCE_OK, FLCE_EINVAL (null array) or FLCE_EDEVICE.
 */
int flce_profile_read(hipStream_t stream, double* total_ms, int64_t* launches, int reset);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H_ */
