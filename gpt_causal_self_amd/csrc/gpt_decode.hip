// gpt_decode.hip -- C ABI of the one-token decode with a key/value cache
// (include/gpt_decode.h).
#include "../../include/gpt_decode.h"
#include "decode.cuh"
#include "handle.cuh"

using namespace gpt_attn;

namespace {

#ifndef GA_DEC_ATTN_THREADS
#define GA_DEC_ATTN_THREADS 1024
#endif
#ifndef GA_DEC_ATTN_KPW
#define GA_DEC_ATTN_KPW 64
#endif
constexpr int kDecAttnThreads = GA_DEC_ATTN_THREADS;
constexpr int kDecAttnKpw = GA_DEC_ATTN_KPW;  // cached keys per wave
constexpr int kDecChunk = kDecAttnThreads / 64 * kDecAttnKpw;
inline int nchunks(int n) { return (n + kDecChunk - 1) / kDecChunk; }

}  // namespace

extern "C" {

int gpt_attn_decode(gpt_attn_t h, const void* x_new, int B, int pos, const void* W_attn,
                    const void* b_attn, const void* W_proj, const void* b_proj, int n_head,
                    void* k_cache, void* v_cache, int cache_T, void* y, void* stream) {
  if (!h || !x_new || !W_attn || !W_proj || !k_cache || !v_cache || !y)
    return GPT_ATTN_ERR_INVALID_ARG;
  if (B < 0 || pos < 0 || cache_T <= 0 || pos >= cache_T) return GPT_ATTN_ERR_INVALID_ARG;
  if (h->dtype != GPT_ATTN_BF16) return GPT_ATTN_ERR_UNSUPPORTED;
  if (n_head != h->H || B > h->max_B) return GPT_ATTN_ERR_SHAPE;
  if (B > kDecMaxB) return GPT_ATTN_ERR_UNSUPPORTED;
  const int C = h->C, H = h->H, hs = h->hs;
  const int nc = nchunks(pos + 1);
  if ((size_t)B * H * nc * (hs + 2) > h->part_elems || B * H > kCounters)
    return GPT_ATTN_ERR_SHAPE;
  if (!aligned16(x_new) || !aligned16(W_attn) || !aligned16(W_proj) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(y) || (b_attn && !aligned16(b_attn)) ||
      (b_proj && !aligned16(b_proj)))
    return GPT_ATTN_ERR_ALIGN;
  h->saved = 0;
  h->last_B = h->last_T = 0;
  if (B == 0) return GPT_ATTN_OK;
  const hipStream_t st = as_stream(stream);
  bf16_t* q = (bf16_t*)h->qkv;  // [B][C]
  bf16_t* ym = (bf16_t*)h->o;   // [B][C]
  float* part = h->part;        // [B*H][nc][hs + 2] attention chunk partials
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hs));
  // arrival counters of the attention's (b, h) blocks (used when the cache
  // spans several chunks)
  unsigned* cnt_attn = h->counters;
  DecQKVOut o1{q, (bf16_t*)k_cache, (bf16_t*)v_cache, C, H, hs, cache_T, pos};
  hipLaunchKernelGGL(skinny_gemm_kernel<DecQKVOut>, dim3((3 * C + kDecCols - 1) / kDecCols),
                     dim3(64 * kDecWaves), skinny_lds_bytes(), st, (const bf16_t*)x_new, B,
                     C, (const bf16_t*)W_attn, 3 * C, (const bf16_t*)b_attn, o1);
  if (hs == 64)
    hipLaunchKernelGGL((decode_attn_kernel<64, kDecAttnThreads, kDecAttnKpw>), dim3(B * H, nc), dim3(kDecAttnThreads), 0, st, q,
                       (const bf16_t*)k_cache, (const bf16_t*)v_cache, part, ym, H, cache_T, pos,
                       nc, scale_log2, cnt_attn);
  else
    hipLaunchKernelGGL((decode_attn_kernel<32, kDecAttnThreads, kDecAttnKpw>), dim3(B * H, nc), dim3(kDecAttnThreads), 0, st, q,
                       (const bf16_t*)k_cache, (const bf16_t*)v_cache, part, ym, H, cache_T, pos,
                       nc, scale_log2, cnt_attn);
  DecRowOut o2{(bf16_t*)y, C};
  hipLaunchKernelGGL(skinny_gemm_kernel<DecRowOut>, dim3((C + kDecCols - 1) / kDecCols),
                     dim3(64 * kDecWaves), skinny_lds_bytes(), st, ym, B, C,
                     (const bf16_t*)W_proj, C, (const bf16_t*)b_proj, o2);
  return launch_status();
}

int gpt_attn_export_kv(gpt_attn_t h, void* k_cache, void* v_cache, int cache_T, void* stream) {
  if (!h || !k_cache || !v_cache || cache_T <= 0) return GPT_ATTN_ERR_INVALID_ARG;
  if (h->dtype != GPT_ATTN_BF16) return GPT_ATTN_ERR_UNSUPPORTED;
  if (h->last_B <= 0 || h->last_T <= 0) return GPT_ATTN_ERR_STATE;
  if (cache_T < h->last_T) return GPT_ATTN_ERR_SHAPE;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return GPT_ATTN_ERR_ALIGN;
  const int B = h->last_B, T = h->last_T, H = h->H, hs = h->hs;
  const size_t head_elems = (size_t)B * H * T * hs;
  const bf16_t* qkv = (const bf16_t*)h->qkv;
  const size_t chunks = head_elems / 8;
  const int grid = (int)((chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096);
  hipLaunchKernelGGL(export_kv_kernel, dim3(grid), dim3(256), 0, as_stream(stream),
                     qkv + head_elems, qkv + 2 * head_elems, (bf16_t*)k_cache, (bf16_t*)v_cache,
                     B * H, T, hs, cache_T);
  return launch_status();
}

}  // extern "C"
