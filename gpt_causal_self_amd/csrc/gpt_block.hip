// gpt_block.hip -- C ABI of the Block pieces around the attention layer
// (include/gpt_block.h): LayerNorm, the Pre-LN attention half-block with its
// residual, and the MLP sublayer with the fused GELU epilogue.
#include "../../include/gpt_block.h"
#include "handle.cuh"
#include "layer_fwd.cuh"
#include "layernorm.cuh"

using namespace gpt_attn;

namespace {

constexpr int kMaxLnC = 8192;

int check_ln(int M, int C) {
  if (M < 0 || C <= 0) return GPT_ATTN_ERR_INVALID_ARG;
  if (C % 8 != 0 || C > kMaxLnC) return GPT_ATTN_ERR_SHAPE;
  return GPT_ATTN_OK;
}

}  // namespace

extern "C" {

int gpt_layernorm(const void* x, int M, int C, const void* w, const void* b, void* out,
                  void* stream) {
  if (!x || !w || !out) return GPT_ATTN_ERR_INVALID_ARG;
  const int rc = check_ln(M, C);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (b && !aligned16(b)))
    return GPT_ATTN_ERR_ALIGN;
  if (M == 0) return GPT_ATTN_OK;
  launch_layernorm((const bf16_t*)x, (const bf16_t*)w, (const bf16_t*)b, (bf16_t*)out, M, C,
                   as_stream(stream));
  return launch_status();
}

int gpt_attn_block_forward(gpt_attn_t h, const void* x, int B, int T, const void* ln_w,
                           const void* ln_b, const void* W_attn, const void* b_attn,
                           const void* W_proj, const void* b_proj, int n_head, void* out,
                           void* stream) {
  if (!h || !x || !ln_w || !W_attn || !W_proj || !out) return GPT_ATTN_ERR_INVALID_ARG;
  if (B < 0 || T < 0) return GPT_ATTN_ERR_INVALID_ARG;
  if (h->dtype != GPT_ATTN_BF16) return GPT_ATTN_ERR_UNSUPPORTED;
  if (n_head != h->H || B > h->max_B || T > h->max_T) return GPT_ATTN_ERR_SHAPE;
  if (h->C % 8 != 0 || h->C > kMaxLnC) return GPT_ATTN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(ln_w) || !aligned16(W_attn) || !aligned16(W_proj) ||
      !aligned16(out) || (ln_b && !aligned16(ln_b)) || (b_attn && !aligned16(b_attn)) ||
      (b_proj && !aligned16(b_proj)))
    return GPT_ATTN_ERR_ALIGN;
  h->saved = 0;  // the workspace no longer holds a plain forward's state
  h->last_B = h->last_T = 0;
  if (B == 0 || T == 0) return GPT_ATTN_OK;
  const hipStream_t st = as_stream(stream);
  const int M = B * T;
  bf16_t* ln = (bf16_t*)h->ln;
  launch_layernorm((const bf16_t*)x, (const bf16_t*)ln_w, (const bf16_t*)ln_b, ln, M, h->C, st);
  const DropParams drop = make_drop(h->drop_p, h->drop_seed);
  layer_forward_bf16(h, ln, B, T, (const bf16_t*)W_attn, (const bf16_t*)b_attn,
                     (const bf16_t*)W_proj, (const bf16_t*)b_proj, (bf16_t*)out,
                     (const bf16_t*)x, nullptr, st, h->drop_p > 0.f ? &drop : nullptr);
  const int rc = launch_status();
  if (rc == GPT_ATTN_OK) {
    h->last_B = B;
    h->last_T = T;
  }
  return rc;
}

int gpt_mlp_forward(const void* x, int M, int C, int F, const void* W_fc, const void* b_fc,
                    const void* W_proj, const void* b_proj, const void* residual, void* hbuf,
                    void* y, void* stream) {
  if (!x || !W_fc || !W_proj || !hbuf || !y) return GPT_ATTN_ERR_INVALID_ARG;
  if (M < 0 || C <= 0 || F <= 0) return GPT_ATTN_ERR_INVALID_ARG;
  if (C % 8 != 0 || F % 8 != 0) return GPT_ATTN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(W_fc) || !aligned16(W_proj) || !aligned16(hbuf) ||
      !aligned16(y) || (b_fc && !aligned16(b_fc)) || (b_proj && !aligned16(b_proj)) ||
      (residual && !aligned16(residual)))
    return GPT_ATTN_ERR_ALIGN;
  if (M == 0) return GPT_ATTN_OK;
  const hipStream_t st = as_stream(stream);
  Epi2Gelu e1{(bf16_t*)hbuf, F, (const bf16_t*)b_fc};
  launch_gemm2<GA_FC_TILE>((const bf16_t*)x, C, (const bf16_t*)W_fc, F, M, F, C, e1, st);
  // c_proj [4C -> C]: the split-role GEMM on 96 x 384 tiles where C allows
  // (csrc/gemm3.cuh), else gemm2
  const bool g3 = use_gemm3(M, C);
  if (residual) {
    Epi2RowMajorRes e2{(bf16_t*)y, C, (const bf16_t*)b_proj, (const bf16_t*)residual};
    if (g3)
      launch_gemm3<GA_PROJ3_TILE, true, false>((const bf16_t*)hbuf, F, (const bf16_t*)W_proj, C,
                                               M, C, F, e2, st);
    else
      launch_gemm2<GA_FCPROJ_TILE>((const bf16_t*)hbuf, F, (const bf16_t*)W_proj, C, M, C, F,
                                   e2, st);
  } else {
    Epi2RowMajor e2{(bf16_t*)y, C, (const bf16_t*)b_proj};
    if (g3)
      launch_gemm3<GA_PROJ3_TILE, true, false>((const bf16_t*)hbuf, F, (const bf16_t*)W_proj, C,
                                               M, C, F, e2, st);
    else
      launch_gemm2<GA_FCPROJ_TILE>((const bf16_t*)hbuf, F, (const bf16_t*)W_proj, C, M, C, F,
                                   e2, st);
  }
  return launch_status();
}

}  // extern "C"
