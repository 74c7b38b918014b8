/*
 * gpt_decode.h -- one-token decode of the causal self-attention layer with a
 * key/value cache, for MI355X (gfx950), bf16 handles only.
 *
 * The pages generate text one token at a time by running the whole
 * (block_size-cropped) prefix through the model and keeping the last
 * position (page "nanoGPT global flow walkthrough" (devpress.csdn.net), fifth
 * stage, GPT.generate); page "GPT architecture: design ideas and core
 * concepts" (paozippq.com), extension directions, names the KV cache as the
 * inference optimisation.  The layer is causal, so its output at position
 * pos depends only on positions 0..pos: one decode step that keeps the keys
 * and values of earlier positions in a cache gives the same row as the full
 * forward over 0..pos (up to rounding order).
 *
 * Cache layout: k_cache and v_cache are caller-owned DEVICE buffers
 * [B][n_head][cache_T][hs] in bf16 (row of position t of head h of sequence
 * b at ((b*n_head + h)*cache_T + t)*hs), 16-byte aligned.  All sequences of a
 * call share the position.  Conventions otherwise as gpt_attn.h.
 */
#ifndef GPT_DECODE_H
#define GPT_DECODE_H

#include <stddef.h>

#include "gpt_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Decode one token per sequence at position pos:
 *   qkv   = x_new . W_attn + b_attn              (x_new [B, C])
 *   k_cache[b][h][pos] = k, v_cache[b][h][pos] = v   (rounded to bf16)
 *   y_m   = softmax_{j <= pos}(q k_j / sqrt(hs)) v_j per head (keys and values
 *           of positions < pos read from the caches)
 *   y     = y_m . W_proj + b_proj                (y [B, C])
 * q/k/v and y_m are rounded to bf16 as in gpt_attn_forward; scores, softmax
 * statistics and the weighted value sum are fp32.  Uses the handle's
 * workspace (a saved forward state is dropped).  B = 0 is a no-op.
 * Errors: INVALID_ARG (NULL pointer, B < 0, pos < 0, cache_T <= 0,
 * pos >= cache_T), SHAPE (n_head differs from the handle's, B > the handle's
 * max_B, B * n_head > 4096, or the per-chunk partials of
 * B * n_head * ceil((pos + 1) / 1024) rows exceed the workspace),
 * UNSUPPORTED (fp32 handle or B > 16),
 * ALIGN, HIP.  Calls that overlap on one handle race (they share its
 * workspace and its arrival counters). */
int gpt_attn_decode(gpt_attn_t h, const void *x_new, int B, int pos, const void *W_attn,
                    const void *b_attn, const void *W_proj, const void *b_proj, int n_head,
                    void *k_cache, void *v_cache, int cache_T, void *y, void *stream);

/* Prefill: copy the keys and values of positions 0..T-1 computed by the last
 * gpt_attn_forward / gpt_attn_block_forward on this handle (B, T of that
 * call) into the caches, so that decoding can continue at pos = T.
 * Errors: INVALID_ARG (NULL pointer, cache_T <= 0), STATE (no forward since
 * the handle was created or since the last decode), SHAPE (cache_T < T),
 * UNSUPPORTED (fp32 handle), ALIGN, HIP. */
int gpt_attn_export_kv(gpt_attn_t h, void *k_cache, void *v_cache, int cache_T, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT_DECODE_H */
