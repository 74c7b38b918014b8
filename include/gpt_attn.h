/*
 * gpt_attn.h -- C ABI of the MI355X (gfx950) causal self-attention layer.
 *
 * The layer is the GPT-2 / nanoGPT CausalSelfAttention forward (page
 * "nanoGPT global flow walkthrough" (devpress.csdn.net), section 2.5 (B);
 * page "nanoGPT architecture explained step by step" (lzwjava.github.io),
 * section 3):
 *
 *   qkv = x . W_attn + b_attn                      c_attn, one fused linear
 *   q, k, v = split(qkv), each viewed as n_head heads of hs = C / n_head
 *   att = softmax(mask(q k^T / sqrt(hs)))          mask: key j visible to
 *                                                  query i iff j <= i
 *   y_m = merge_heads(att v)
 *   y   = y_m . W_proj + b_proj                    c_proj
 *
 * Dropout is the identity by default (dropout 0.0 in GPTConfig, page
 * "nanoGPT global flow walkthrough", section 2.1); gpt_attn_set_dropout
 * switches on the training-time dropout.
 *
 * Conventions for every entry point:
 *   - Tensors are row-major and contiguous.  Weights are [in, out]
 *     (y = x . W), i.e. the transpose of nn.Linear's [out, in] storage.
 *   - Tensor pointers are DEVICE pointers on the handle's device, owned by
 *     the caller, 16-byte aligned, and in the handle's element type
 *     (GPT_ATTN_F32: float; GPT_ATTN_BF16: bfloat16 bit patterns).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: they return after enqueueing kernels; faults during
 *     execution surface on the caller's next synchronisation.
 *   - Every argument is validated on the host before any device call, so an
 *     argument error never touches the device.
 *   - A handle is not thread-safe; calls that overlap on one handle race.
 *   - The bf16 path accumulates in fp32, keeps softmax statistics in fp32 and
 *     rounds every bf16 store to nearest-even.
 */
#ifndef GPT_ATTN_H
#define GPT_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
enum gpt_attn_status {
  GPT_ATTN_OK = 0,
  GPT_ATTN_ERR_INVALID_ARG = 1, /* NULL pointer, non-positive size, bad dtype   */
  GPT_ATTN_ERR_SHAPE = 2,       /* C % n_head != 0, n_head mismatch, B/T > max,
                                   or above the allocation-free scratch        */
  GPT_ATTN_ERR_UNSUPPORTED = 3, /* head size other than 32 or 64                */
  GPT_ATTN_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned      */
  GPT_ATTN_ERR_OOM = 5,         /* workspace allocation failed                  */
  GPT_ATTN_ERR_HIP = 6,         /* a HIP runtime call or a launch failed        */
  GPT_ATTN_ERR_STATE = 7        /* backward without a matching saved forward    */
};

/* Element types. */
enum gpt_attn_dtype { GPT_ATTN_F32 = 0, GPT_ATTN_BF16 = 1 };

typedef struct gpt_attn_handle *gpt_attn_t;

/* Bytes of device workspace a handle created with these arguments owns.
 * Host-only; never touches the device.  Returns INVALID_ARG / SHAPE /
 * UNSUPPORTED like gpt_attn_create. */
int gpt_attn_workspace_bytes(int C, int n_head, int max_B, int max_T, int dtype,
                             size_t *bytes);

/* Create a layer handle for embedding size C (n_embd) and n_head heads
 * (GPTConfig fields n_embd and n_head; the module asserts
 * n_embd % n_head == 0, page "nanoGPT architecture explained step by step",
 * section 3).  max_B and max_T bound the batch and sequence length of later
 * calls (T plays the role of block_size: the mask buffer there is sliced to
 * T x T).  Allocates the workspace on the current device (intermediate q, k,
 * v, merged heads, softmax log-sum-exp and backward scratch).
 * Errors: INVALID_ARG (out NULL, C/n_head/max_B/max_T <= 0, bad dtype),
 * SHAPE (C % n_head != 0), UNSUPPORTED (hs not in {32, 64}), OOM, HIP.
 * On error *out is set to NULL. */
int gpt_attn_create(gpt_attn_t *out, int C, int n_head, int max_B, int max_T,
                    int dtype);

/* Forward of the layer.
 *   x      [B, T, C]       input (in the model: ln_1 of the residual stream)
 *   W_attn [C, 3C]         c_attn weight; columns [0,C) give q, [C,2C) k,
 *                          [2C,3C) v; head h owns columns [h*hs,(h+1)*hs)
 *                          of each block
 *   b_attn [3C] or NULL    c_attn bias (NULL = bias=False)
 *   W_proj [C, C]          c_proj weight
 *   b_proj [C] or NULL     c_proj bias (NULL = bias=False)
 *   n_head                 must equal the handle's
 *   y      [B, T, C]       output; must not overlap any input
 *   save_for_backward      non-zero: keep q, k, v, the merged heads and the
 *                          softmax log-sum-exp in the workspace for
 *                          gpt_attn_backward
 * B = 0 or T = 0 is a no-op.  Errors: INVALID_ARG, SHAPE (n_head differs
 * from the handle's, B > max_B, T > max_T), ALIGN, HIP. */
int gpt_attn_forward(gpt_attn_t h, const void *x, int B, int T,
                     const void *W_attn, const void *b_attn, const void *W_proj,
                     const void *b_proj, int n_head, void *y, void *stream,
                     int save_for_backward);

/* Exact gradient of the layer (the chain rule through the steps above; the
 * pages leave the backward to autograd, page "nanoGPT global flow
 * walkthrough", section 3).  Requires that the last forward on this handle
 * ran with save_for_backward != 0 and the same B and T, else STATE.
 *   dY      [B, T, C]      upstream gradient of y
 *   dx      [B, T, C]      out: gradient of x
 *   dW_attn [C, 3C], dW_proj [C, C]   out: weight gradients
 *   db_attn [3C], db_proj [C]          out, or NULL when the layer has no
 *                                      bias (then they are not computed)
 * Gradients are overwritten, not accumulated, in the handle's dtype.
 * Errors: INVALID_ARG, SHAPE, ALIGN, STATE, HIP. */
int gpt_attn_backward(gpt_attn_t h, const void *x, const void *W_attn,
                      const void *W_proj, const void *dY, void *dx,
                      void *dW_attn, void *db_attn, void *dW_proj,
                      void *db_proj, int B, int T, void *stream);

/* Dropout for the following forwards on this handle (training): nn.Dropout
 * on the attention weights after the softmax and on the c_proj output, rate
 * p = config.dropout (page "nanoGPT architecture explained step by step",
 * section 3, attn_dropout and resid_dropout).  p = 0 (the default) is the
 * identity.  Masks come from the Philox4x32-10 counter-based generator
 * (Salmon et al., SC 2011) keyed by seed (low word, high word): attention
 * weight (b, h, query i, key j) uses counter (j/8, i, b*n_head + h, 1) and
 * the 16-bit half j%2 (0: low) of output word (j%8)/2, dropped iff that half
 * is below floor(p * 2^16) (capped at 2^16 - 1); c_proj output (row
 * m = b*T + t, column n) uses counter (n/4, m, 0, 2) and word n%4, dropped
 * iff that word is below floor(p * 2^32); kept elements are scaled by
 * 1/(1-p).  The softmax row is
 * normalised over all visible keys before dropping.  A forward with
 * save_for_backward records p and seed, and gpt_attn_backward then returns
 * the exact gradient through the same masks (the upstream gradient of the
 * c_proj output is masked, rescaled and stored in bf16 before the c_proj
 * gradients).  Callers change the seed between steps.
 * Such a forward also stores the attention weights' keep decisions, one bit
 * per weight in two layouts, which the backward reads instead of drawing the
 * generator again; the first call with p > 0 allocates that buffer on the
 * handle's device, max_B*n_head*2*R*(ceil(max_T/64) + R/64)*4 bytes with
 * R = max_T rounded up to 128 (37.7 MB at max_B 12, n_head 12, max_T 1024),
 * freed by gpt_attn_destroy.
 * Applies to gpt_attn_forward and gpt_attn_block_forward (bf16), not to
 * decoding.  Errors: INVALID_ARG (NULL handle, p < 0, p >= 1 or NaN),
 * UNSUPPORTED (p > 0 on an fp32 handle), OOM or HIP (that buffer; dropout
 * then stays as it was). */
int gpt_attn_set_dropout(gpt_attn_t h, float p, unsigned long long seed);

/* Release the handle and its workspace (waits for the device first).
 * NULL is a no-op.  Returns OK or HIP. */
int gpt_attn_destroy(gpt_attn_t h);

/* Measurement hook.  `events` points to n hipEvent_t created by the caller
 * (or is NULL to switch recording off).  With n >= 4 every later forward
 * records events[0] before the c_attn GEMM, events[1] after it, events[2]
 * after the attention kernel and events[3] after c_proj, on the forward's
 * stream; with n >= 8 every later backward also records events[4] before its
 * first kernel, events[5] after the c_proj gradient stage, events[6] after
 * the attention gradient stage and events[7] after the c_attn gradient
 * stage.  The handle keeps a copy of the first min(n, 8) handles; the caller
 * owns the events and must keep them alive while recording is on.
 * Errors: INVALID_ARG (NULL handle, or events non-NULL with n < 4). */
int gpt_attn_set_stage_events(gpt_attn_t h, void *const *events, int n);

/* Bytes of the static device scratch of gpt_attn_forward_noalloc. */
#define GPT_ATTN_NOALLOC_SCRATCH_BYTES (80u << 20)

/* Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Computes what gpt_attn_forward computes on a bf16 handle with
 * dropout off and no state kept for a backward (the same kernels), without a
 * handle and without any allocation: the intermediates (q, k, v, the merged
 * heads, split-K partial sums of short sequences) live in a static device
 * array of GPT_ATTN_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * every GPU it has run on until the process ends.  Element type bf16;
 * tensors and their layouts as in gpt_attn_forward, on the current device;
 * C = n_embd.  The array keeps the last call's contents; every call on one
 * GPU uses the same array, so calls that overlap on one GPU (on different
 * streams or from several host threads) race.  B = 0 or T = 0 is a no-op.
 * Errors: INVALID_ARG (NULL tensor, negative or non-positive size),
 * SHAPE (C % n_head != 0, or the intermediates -- 3*B*T*C and B*T*C bf16
 * values, each rounded up to 256 bytes -- exceed
 * GPT_ATTN_NOALLOC_SCRATCH_BYTES; the GPT-2 124M workload B = 12, T = 1024,
 * C = 768 needs 75.5 MB), UNSUPPORTED (hs not in {32, 64}), ALIGN, HIP. */
int gpt_attn_forward_noalloc(const void *x, int B, int T, int C, int n_head,
                             const void *W_attn, const void *b_attn,
                             const void *W_proj, const void *b_proj, void *y,
                             void *stream);

/* Static description of a status code (never NULL). */
const char *gpt_attn_strerror(int code);

/* Test access to the intermediates of the last forward, in the workspace
 * (device pointers, valid until the next call on the handle):
 *   qkv [3][B][H][T][hs]  q, k, v head-major, handle dtype
 *   o   [B][T][C]         merged heads before c_proj, handle dtype
 *   lse [B][H][T]         float natural-log log-sum-exp of each softmax row
 *                         (written only by a forward with save_for_backward)
 * Any output pointer may be NULL.  Errors: INVALID_ARG. */
int gpt_attn_debug_workspace(gpt_attn_t h, const void **qkv, const void **o,
                             const void **lse);

/* Test access to the intermediates of the last backward (device pointers,
 * valid until the next call on the handle):
 *   dym   [B][T][C]   gradient of the merged heads, handle dtype
 *   dqkv  [B][T][3C]  gradient of the c_attn output (q, k, v blocks),
 *                     handle dtype
 *   delta [B][H][T]   float rowsum(dO * O) of every softmax row
 * Any output pointer may be NULL.  Errors: INVALID_ARG. */
int gpt_attn_debug_backward(gpt_attn_t h, const void **dym, const void **dqkv,
                            const void **delta);

#ifdef __cplusplus
}
#endif

#endif /* GPT_ATTN_H */
