/*
 * gpt_block.h -- C ABI of the pieces of a GPT-2 / nanoGPT Block around the
 * causal self-attention layer, for MI355X (gfx950), bf16 only.
 *
 * The Block is Pre-LN with residual connections (page "nanoGPT global flow
 * walkthrough" (devpress.csdn.net), section 2.5, Block.forward and (A);
 * page "nanoGPT architecture explained step by step" (lzwjava.github.io),
 * section 2):
 *
 *   x = x + attn(ln_1(x))          gpt_attn_block_forward
 *   x = x + mlp(ln_2(x))           gpt_layernorm + gpt_mlp_forward
 *
 *   LayerNorm(u) = (u - mean(u)) / sqrt(var(u) + 1e-5) * w + b over the C
 *                  features of each token, var the biased (population)
 *                  variance, as F.layer_norm (page "nanoGPT global flow
 *                  walkthrough", section 2.5 (A))
 *   mlp(u)       = gelu(u . W_fc + b_fc) . W_proj + b_proj, with the exact
 *                  GELU g(v) = v * Phi(v), Phi the standard normal CDF
 *                  (page "nanoGPT architecture explained step by step",
 *                  section 4; page "nanoGPT global flow walkthrough",
 *                  section 2.5 (C)); dropout is the identity (dropout 0.0).
 *
 * Conventions (as gpt_attn.h): row-major contiguous tensors, weights stored
 * [in, out]; DEVICE pointers owned by the caller, 16-byte aligned, bfloat16
 * bit patterns; `stream` a hipStream_t (NULL = default stream); calls are
 * asynchronous and validate every argument on the host before any device
 * call.  Arithmetic is fp32 (LayerNorm statistics, GEMM accumulation, GELU)
 * and every bf16 store rounds to nearest-even.  Status codes are those of
 * gpt_attn.h.
 */
#ifndef GPT_BLOCK_H
#define GPT_BLOCK_H

#include <stddef.h>

#include "gpt_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* LayerNorm of M rows of C features:
 *   out[m][c] = (x[m][c] - mu_m) * rsqrt(var_m + 1e-5) * w[c] + b[c]
 * with mu_m and var_m (biased) the mean and variance of row m.
 *   x [M, C], out [M, C] (may not overlap x), w [C], b [C] or NULL (no shift).
 * C must be a multiple of 8 and at most 8192.  M = 0 is a no-op.
 * Errors: INVALID_ARG (NULL pointer, M < 0, C <= 0), SHAPE (C % 8 != 0 or
 * C > 8192), ALIGN, HIP. */
int gpt_layernorm(const void *x, int M, int C, const void *w, const void *b, void *out,
                  void *stream);

/* Attention half of a Block: out = x + attn(ln_1(x)), on a bf16 handle.
 *   x [B, T, C]; ln_w [C], ln_b [C] or NULL: ln_1 weight and bias;
 *   W_attn, b_attn, W_proj, b_proj, n_head: as gpt_attn_forward;
 *   out [B, T, C], must not overlap x or the weights.
 * ln_1(x) is rounded to bf16 into the handle's workspace and then goes
 * through the layer exactly as gpt_attn_forward's x; the residual x is added
 * to the c_proj accumulator (with b_proj) before the single rounding of out.
 * B = 0 or T = 0 is a no-op.  Does not keep state for gpt_attn_backward.
 * Errors: as gpt_attn_forward, plus UNSUPPORTED for an fp32 handle. */
int gpt_attn_block_forward(gpt_attn_t h, const void *x, int B, int T, const void *ln_w,
                           const void *ln_b, const void *W_attn, const void *b_attn,
                           const void *W_proj, const void *b_proj, int n_head, void *out,
                           void *stream);

/* MLP sublayer (c_fc -> GELU -> c_proj) over M token rows, optionally with
 * the Block's residual add:
 *   hbuf = bf16(gelu(x . W_fc + b_fc))                       [M, F]
 *   y    = bf16(hbuf . W_proj + b_proj (+ residual))          [M, C]
 *   x [M, C]; W_fc [C, F]; b_fc [F] or NULL; W_proj [F, C]; b_proj [C] or
 *   NULL; residual [M, C] or NULL; hbuf [M, F]: caller-owned scratch that
 *   receives the activations; y [M, C] must not overlap x, hbuf or residual
 *   (y == residual is not allowed either).
 * GELU is applied to the fp32 accumulator plus bias before the rounding of
 * hbuf.  C and F must be multiples of 8.  M = 0 is a no-op.
 * Errors: INVALID_ARG (NULL required pointer, M < 0, C or F <= 0), SHAPE
 * (C or F not a multiple of 8), ALIGN, HIP. */
int gpt_mlp_forward(const void *x, int M, int C, int F, const void *W_fc, const void *b_fc,
                    const void *W_proj, const void *b_proj, const void *residual, void *hbuf,
                    void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT_BLOCK_H */
