// gpt_attn.hip -- C ABI of the causal self-attention layer (include/gpt_attn.h).
//
// Host side: argument validation (always before any device call), workspace
// ownership, and the launch sequence on the caller's stream:
//   forward : c_attn GEMM (bias + head-major q/k/v scatter)
//             -> fused causal attention (merged-head output, optional LSE)
//             -> c_proj GEMM (bias)
//   backward: see attn_bwd.cuh / the launch sequence in gpt_attn_backward.
#include <algorithm>

#include "attn_bwd.cuh"
#include "attn_bwd2.cuh"
#include "handle.cuh"
#include "layer_fwd.cuh"

using namespace gpt_attn;

extern "C" {

const char* gpt_attn_strerror(int code) {
  switch (code) {
    case GPT_ATTN_OK: return "ok";
    case GPT_ATTN_ERR_INVALID_ARG: return "invalid argument (NULL pointer, non-positive size or unknown dtype)";
    case GPT_ATTN_ERR_SHAPE: return "shape error (C % n_head != 0, n_head mismatch, B/T above the handle's maximum, or intermediates larger than the allocation-free forward's static scratch)";
    case GPT_ATTN_ERR_UNSUPPORTED: return "unsupported configuration (head size must be 32 or 64)";
    case GPT_ATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case GPT_ATTN_ERR_OOM: return "device workspace allocation failed";
    case GPT_ATTN_ERR_HIP: return "HIP runtime or kernel launch error";
    case GPT_ATTN_ERR_STATE: return "backward needs a preceding forward with save_for_backward and the same B, T";
    default: return "unknown status code";
  }
}

int gpt_attn_workspace_bytes(int C, int n_head, int max_B, int max_T, int dtype,
                             size_t* bytes) {
  if (!bytes) return GPT_ATTN_ERR_INVALID_ARG;
  const int rc = check_dims(C, n_head, max_B, max_T, dtype);
  if (rc) return rc;
  *bytes = layout(C, n_head, max_B, max_T, dtype == GPT_ATTN_F32 ? 4 : 2).total;
  return GPT_ATTN_OK;
}

int gpt_attn_create(gpt_attn_t* out, int C, int n_head, int max_B, int max_T, int dtype) {
  if (!out) return GPT_ATTN_ERR_INVALID_ARG;
  *out = nullptr;
  const int rc = check_dims(C, n_head, max_B, max_T, dtype);
  if (rc) return rc;
  gpt_attn_handle* h = (gpt_attn_handle*)calloc(1, sizeof(gpt_attn_handle));
  if (!h) return GPT_ATTN_ERR_OOM;
  h->C = C;
  h->H = n_head;
  h->hs = C / n_head;
  h->max_B = max_B;
  h->max_T = max_T;
  h->dtype = dtype;
  h->esize = dtype == GPT_ATTN_F32 ? 4 : 2;
  const Layout L = layout(C, n_head, max_B, max_T, h->esize);
  if (hipGetDevice(&h->device) != hipSuccess) {
    free(h);
    return GPT_ATTN_ERR_HIP;
  }
  void* ws = nullptr;
  const hipError_t e = hipMalloc(&ws, L.total);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    free(h);
    return e == hipErrorOutOfMemory ? GPT_ATTN_ERR_OOM : GPT_ATTN_ERR_HIP;
  }
  h->ws = (char*)ws;
  h->ws_bytes = L.total;
  h->qkv = h->ws + L.qkv;
  h->o = h->ws + L.o;
  h->lse = (float*)(h->ws + L.lse);
  h->dym = h->ws + L.dym;
  h->dqkv = h->ws + L.dqkv;
  h->delta = (float*)(h->ws + L.delta);
  h->part = (float*)(h->ws + L.part);
  h->part_elems = L.part_elems;
  h->ln = h->ws + L.ln;
  h->rowstats = (float*)(h->ws + L.rowstats);
  h->counters = (unsigned*)(h->ws + L.counters);
  if (hipMemset(h->counters, 0, kCounters * sizeof(unsigned)) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess ||
      hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(ws);
    free(h);
    return GPT_ATTN_ERR_HIP;
  }
  if (hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
    (void)hipStreamDestroy(h->side);
    (void)hipFree(ws);
    free(h);
    return GPT_ATTN_ERR_HIP;
  }

  *out = h;
  return GPT_ATTN_OK;
}

int gpt_attn_destroy(gpt_attn_t h) {
  if (!h) return GPT_ATTN_OK;
  int rc = GPT_ATTN_OK;
  if (h->ws) {
    if (hipDeviceSynchronize() != hipSuccess) rc = GPT_ATTN_ERR_HIP;
    if (hipFree(h->ws) != hipSuccess) rc = GPT_ATTN_ERR_HIP;
  }
  if (h->keepq && hipFree(h->keepq) != hipSuccess) rc = GPT_ATTN_ERR_HIP;
  if (h->ev_fork && hipEventDestroy(h->ev_fork) != hipSuccess) rc = GPT_ATTN_ERR_HIP;
  if (h->ev_join && hipEventDestroy(h->ev_join) != hipSuccess) rc = GPT_ATTN_ERR_HIP;
  if (h->side && hipStreamDestroy(h->side) != hipSuccess) rc = GPT_ATTN_ERR_HIP;
  free(h);
  return rc;
}

int gpt_attn_debug_backward(gpt_attn_t h, const void** dym, const void** dqkv,
                            const void** delta) {
  if (!h) return GPT_ATTN_ERR_INVALID_ARG;
  if (dym) *dym = h->dym;
  if (dqkv) *dqkv = h->dqkv;
  if (delta) *delta = h->delta;
  return GPT_ATTN_OK;
}

int gpt_attn_set_stage_events(gpt_attn_t h, void* const* events, int n) {
  if (!h) return GPT_ATTN_ERR_INVALID_ARG;
  if (!events) {
    h->n_ev = 0;
    return GPT_ATTN_OK;
  }
  if (n < 4) return GPT_ATTN_ERR_INVALID_ARG;
  h->n_ev = n < 8 ? 4 : 8;
  for (int i = 0; i < h->n_ev; ++i) h->ev[i] = (hipEvent_t)events[i];
  return GPT_ATTN_OK;
}

int gpt_attn_debug_workspace(gpt_attn_t h, const void** qkv, const void** o,
                             const void** lse) {
  if (!h) return GPT_ATTN_ERR_INVALID_ARG;
  if (qkv) *qkv = h->qkv;
  if (o) *o = h->o;
  if (lse) *lse = h->lse;
  return GPT_ATTN_OK;
}

int gpt_attn_forward(gpt_attn_t h, const void* x, int B, int T, const void* W_attn,
                     const void* b_attn, const void* W_proj, const void* b_proj,
                     int n_head, void* y, void* stream, int save_for_backward) {
  // ---- validation (host only)
  if (!h || !x || !W_attn || !W_proj || !y) return GPT_ATTN_ERR_INVALID_ARG;
  if (B < 0 || T < 0) return GPT_ATTN_ERR_INVALID_ARG;
  if (n_head != h->H || B > h->max_B || T > h->max_T) return GPT_ATTN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(W_attn) || !aligned16(W_proj) || !aligned16(y) ||
      (b_attn && !aligned16(b_attn)) || (b_proj && !aligned16(b_proj)))
    return GPT_ATTN_ERR_ALIGN;
  h->saved = 0;
  h->last_B = h->last_T = 0;
  if (B == 0 || T == 0) {  // nothing to compute; an empty backward may follow
    if (save_for_backward) {
      h->saved = 1;
      h->saved_B = B;
      h->saved_T = T;
    }
    return GPT_ATTN_OK;
  }

  const int C = h->C, H = h->H, hs = h->hs;
  const int M = B * T;
  const hipStream_t st = as_stream(stream);
  const size_t head_elems = (size_t)B * H * T * hs;  // one of q, k, v
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hs));
  float* lse = save_for_backward ? h->lse : nullptr;
  (void)M;

  if (h->dtype == GPT_ATTN_BF16) {
    const DropParams drop = make_drop(h->drop_p, h->drop_seed);
    const bool keep = h->drop_p > 0.f && save_for_backward;
    layer_forward_bf16(h, (const bf16_t*)x, B, T, (const bf16_t*)W_attn, (const bf16_t*)b_attn,
                       (const bf16_t*)W_proj, (const bf16_t*)b_proj, (bf16_t*)y, nullptr, lse,
                       st, h->drop_p > 0.f ? &drop : nullptr, keep ? h->keepq : nullptr,
                       keep ? h->keepk : nullptr);
  } else {
    const float* xf = (const float*)x;
    float* qkv = (float*)h->qkv;
    float* o = (float*)h->o;
    EpiQKV<float> e1{qkv, (const float*)b_attn, B, T, C, H, hs};
    mark(h, 0, st);
    launch_gemm_f32<true, false>(xf, C, (const float*)W_attn, 3 * C, M, 3 * C, C, e1, st);
    mark(h, 1, st);
    const dim3 agrid(B * H, (T + 63) / 64);
    if (hs == 64)
      hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, agrid, dim3(256), 0, st, qkv,
                         qkv + head_elems, qkv + 2 * head_elems, o, lse, H, T, scale_log2);
    else
      hipLaunchKernelGGL(attn_fwd_f32_kernel<32>, agrid, dim3(256), 0, st, qkv,
                         qkv + head_elems, qkv + 2 * head_elems, o, lse, H, T, scale_log2);
    mark(h, 2, st);
    EpiRowMajor<float> e3{(float*)y, C, (const float*)b_proj};
    launch_gemm_f32<true, false>(o, C, (const float*)W_proj, C, M, C, C, e3, st);
    mark(h, 3, st);
  }
  const int rc = launch_status();
  h->last_B = rc == GPT_ATTN_OK ? B : 0;
  h->last_T = rc == GPT_ATTN_OK ? T : 0;
  if (rc == GPT_ATTN_OK && save_for_backward) {
    h->saved = 1;
    h->saved_B = B;
    h->saved_T = T;
    h->saved_drop_p = h->drop_p;
    h->saved_drop_seed = h->drop_seed;
  }
  return rc;
}

int gpt_attn_set_dropout(gpt_attn_t h, float p, unsigned long long seed) {
  if (!h || !(p >= 0.f && p < 1.f)) return GPT_ATTN_ERR_INVALID_ARG;
  if (p > 0.f && h->dtype != GPT_ATTN_BF16) return GPT_ATTN_ERR_UNSUPPORTED;
  if (p > 0.f && !h->keepq) {
    const KeepBitsLayout kl(h->max_T);
    const size_t bh = (size_t)h->max_B * h->H;
    const size_t qb = align_up(kl.q_words((int)bh) * sizeof(uint32_t));
    const size_t kb = kl.k_words((int)bh) * sizeof(uint32_t);
    void* buf = nullptr;
    const hipError_t e = hipMalloc(&buf, qb + kb);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return e == hipErrorOutOfMemory ? GPT_ATTN_ERR_OOM : GPT_ATTN_ERR_HIP;
    }
    h->keepq = (uint32_t*)buf;
    h->keepk = (uint16_t*)((char*)buf + qb);
  }
  h->drop_p = p;
  h->drop_seed = seed;
  return GPT_ATTN_OK;
}

int gpt_attn_backward(gpt_attn_t h, const void* x, const void* W_attn, const void* W_proj,
                      const void* dY, void* dx, void* dW_attn, void* db_attn, void* dW_proj,
                      void* db_proj, int B, int T, void* stream) {
  // ---- validation (host only)
  if (!h || !x || !W_attn || !W_proj || !dY || !dx || !dW_attn || !dW_proj)
    return GPT_ATTN_ERR_INVALID_ARG;
  if (B < 0 || T < 0) return GPT_ATTN_ERR_INVALID_ARG;
  if (B > h->max_B || T > h->max_T) return GPT_ATTN_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(W_attn) || !aligned16(W_proj) || !aligned16(dY) ||
      !aligned16(dx) || !aligned16(dW_attn) || !aligned16(dW_proj) ||
      (db_attn && !aligned16(db_attn)) || (db_proj && !aligned16(db_proj)))
    return GPT_ATTN_ERR_ALIGN;
  if (!h->saved || h->saved_B != B || h->saved_T != T) return GPT_ATTN_ERR_STATE;

  const int C = h->C, H = h->H, hs = h->hs;
  const int M = B * T, N3 = 3 * C;
  const hipStream_t st = as_stream(stream);
  const float scale = (float)(1.0 / sqrt((double)hs));
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hs));
  const size_t head_elems = (size_t)B * H * T * hs;
  float* part = h->part;                                   // split-K partials
  float* cpart = h->part + (size_t)kWgradSplits * (C + 1) * N3;  // column-sum partials
  const int rows_per = (M + kColsumSplits - 1) / kColsumSplits;
  const int ncs = rows_per > 0 ? (M + rows_per - 1) / rows_per : 0;
  // Split-K factor of a weight-gradient GEMM: as many k-slices as fit the
  // chip in one pass (two 128x128 blocks per CU on 256 CUs), so no block
  // waits for a second round.
  auto splits_for = [](int tiles) {
    int s = (2 * 256) / tiles;
    return s < 1 ? 1 : (s > kWgradSplits ? kWgradSplits : s);
  };
  const int rblocks = 1024;

  if (M == 0) {  // empty batch: the weight and bias gradients are zero sums
    const size_t nwa = (size_t)C * N3, nwp = (size_t)C * C;
    if (h->dtype == GPT_ATTN_BF16) {
      hipLaunchKernelGGL(reduce_partials_kernel<bf16_t>, dim3(rblocks), dim3(256), 0, st, part,
                         0, nwa, nwa, (bf16_t*)dW_attn);
      hipLaunchKernelGGL(reduce_partials_kernel<bf16_t>, dim3(rblocks), dim3(256), 0, st, part,
                         0, nwp, nwp, (bf16_t*)dW_proj);
      if (db_attn)
        hipLaunchKernelGGL(reduce_partials_kernel<bf16_t>, dim3(16), dim3(256), 0, st, part, 0,
                           (size_t)N3, (size_t)N3, (bf16_t*)db_attn);
      if (db_proj)
        hipLaunchKernelGGL(reduce_partials_kernel<bf16_t>, dim3(16), dim3(256), 0, st, part, 0,
                           (size_t)C, (size_t)C, (bf16_t*)db_proj);
    } else {
      hipLaunchKernelGGL(reduce_partials_kernel<float>, dim3(rblocks), dim3(256), 0, st, part, 0,
                         nwa, nwa, (float*)dW_attn);
      hipLaunchKernelGGL(reduce_partials_kernel<float>, dim3(rblocks), dim3(256), 0, st, part, 0,
                         nwp, nwp, (float*)dW_proj);
      if (db_attn)
        hipLaunchKernelGGL(reduce_partials_kernel<float>, dim3(16), dim3(256), 0, st, part, 0,
                           (size_t)N3, (size_t)N3, (float*)db_attn);
      if (db_proj)
        hipLaunchKernelGGL(reduce_partials_kernel<float>, dim3(16), dim3(256), 0, st, part, 0,
                           (size_t)C, (size_t)C, (float*)db_proj);
    }
    return launch_status();
  }

  mark(h, 4, st);
  if (h->dtype == GPT_ATTN_BF16) {
    const bf16_t* qkv = (const bf16_t*)h->qkv;
    const bf16_t* o = (const bf16_t*)h->o;
    bf16_t* dym = (bf16_t*)h->dym;
    bf16_t* dqkv = (bf16_t*)h->dqkv;
    // dropout of the saved forward: the c_proj gradients see the masked,
    // rescaled upstream gradient (kept in the ln_1 buffer, unused here)
    const bool drop = h->saved_drop_p > 0.f;
    const DropParams dp = make_drop(h->saved_drop_p, h->saved_drop_seed);
    if (drop) {
      const long groups = (long)M * (C / 4);
      hipLaunchKernelGGL(dropout_grad_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256),
                         0, st, (const bf16_t*)dY, (bf16_t*)h->ln, (long)M, C, dp);
      dY = h->ln;
    }
    // The c_proj weight and bias gradients go to the handle's side stream,
    // forked here (dY and o ready), where they run beside the dO product and
    // the attention backward; the side stream is joined back into st once
    // dqkv is ready, before the c_attn weight gradient reuses the split-K
    // partials (which carry the bias column sums).  Running the c_attn
    // weight gradient on the side stream too, beside the dx product, gained
    // nothing over running the two in sequence and cost one more fork.
    (void)hipEventRecord(h->ev_fork, st);
    // ---- c_proj: dym = dY W_proj^T (its epilogue also writes the softmax
    // backward row statistics D and L) ; dW_proj = ym^T dY ; db_proj = colsum(dY)
    const int Tpad = (T + 63) / 64 * 64;
    float* Dpad = h->rowstats;
    float* Lpad = h->rowstats + (size_t)B * H * Tpad;
    auto dgrad_rowstats = [&](auto e_dym) {
      if (use_gemm3(M, C))
        launch_gemm3<GA_DGRAD3_TILE, true, true>((const bf16_t*)dY, C, (const bf16_t*)W_proj, C,
                                                 M, C, C, e_dym, st);
      else
        launch_gemm2<GA_DGRAD_TILE, true, true>((const bf16_t*)dY, C, (const bf16_t*)W_proj, C,
                                                M, C, C, e_dym, st);
    };
    if (hs == 64)
      dgrad_rowstats(Epi2DgradRowStats<64>{dym, C, nullptr, o, h->lse, Dpad, Lpad, T, H, Tpad});
    else
      dgrad_rowstats(Epi2DgradRowStats<32>{dym, C, nullptr, o, h->lse, Dpad, Lpad, T, H, Tpad});
    // the weight and bias gradients of c_proj need only dY and o: side stream
    const hipStream_t sd = h->side;
    (void)hipStreamWaitEvent(sd, h->ev_fork, 0);
    // db_proj = colsum(dY) comes with the GEMM (row C of each slice's
    // partials, Epi2PartialCS) and is reduced with it
    Epi2PartialCS e_wp{part, C, (size_t)(C + 1) * C, C, db_proj ? 1 : 0};
    const int s1 = splits_for(((C + 127) / 128) * ((C + 127) / 128));
    const int n1 = launch_gemm2<GA_WGRAD_TILE, false, false>(o, C, (const bf16_t*)dY, C, C, C, M,
                                                             e_wp, sd, s1);
    hipLaunchKernelGGL(reduce_partials4_bf16_kernel, dim3(rblocks), dim3(256), 0, sd, part, n1,
                       (size_t)C * C, (size_t)(C + 1) * C, (bf16_t*)dW_proj,
                       db_proj ? (size_t)C : 0, (bf16_t*)db_proj);
    (void)hipEventRecord(h->ev_join, sd);
    mark(h, 5, st);
    // ---- attention core
    const bf16_t* q = qkv;
    const bf16_t* k = qkv + head_elems;
    const bf16_t* v = qkv + 2 * head_elems;
    const dim3 kgrid2(B * H, (T + 127) / 128);
    const dim3 qgrid2(B * H, (T + 127) / 128);
    if (hs == 64) {
      if (drop) {
        hipLaunchKernelGGL((attn_bwd_dkdv2_bf16_kernel<64, true>), kgrid2, dim3(256), 0, st, q,
                           k, v, dym, Lpad, Dpad, dqkv, H, T, Tpad, scale, scale_log2, dp,
                           (const uint32_t*)h->keepk);
        hipLaunchKernelGGL((attn_bwd_dq2_bf16_kernel<64, true>), qgrid2, dim3(256), 0, st, q, k,
                           v, dym, Lpad, Dpad, dqkv, H, T, Tpad, scale, scale_log2, dp,
                           (const uint32_t*)h->keepq);
      } else {
        hipLaunchKernelGGL((attn_bwd_dkdv2_bf16_kernel<64, false>), kgrid2, dim3(256), 0, st, q,
                           k, v, dym, Lpad, Dpad, dqkv, H, T, Tpad, scale, scale_log2,
                           DropParams{}, nullptr);
        hipLaunchKernelGGL((attn_bwd_dq2_bf16_kernel<64, false>), qgrid2, dim3(256), 0, st, q, k,
                           v, dym, Lpad, Dpad, dqkv, H, T, Tpad, scale, scale_log2, DropParams{},
                           nullptr);
      }
    } else {
      if (drop) {
        hipLaunchKernelGGL((attn_bwd_dkdv2_bf16_kernel<32, true>), kgrid2, dim3(256), 0, st, q,
                           k, v, dym, Lpad, Dpad, dqkv, H, T, Tpad, scale, scale_log2, dp,
                           (const uint32_t*)h->keepk);
        hipLaunchKernelGGL((attn_bwd_dq2_bf16_kernel<32, true>), qgrid2, dim3(256), 0, st, q, k,
                           v, dym, Lpad, Dpad, dqkv, H, T, Tpad, scale, scale_log2, dp,
                           (const uint32_t*)h->keepq);
      } else {
        hipLaunchKernelGGL((attn_bwd_dkdv2_bf16_kernel<32, false>), kgrid2, dim3(256), 0, st, q,
                           k, v, dym, Lpad, Dpad, dqkv, H, T, Tpad, scale, scale_log2,
                           DropParams{}, nullptr);
        hipLaunchKernelGGL((attn_bwd_dq2_bf16_kernel<32, false>), qgrid2, dim3(256), 0, st, q, k,
                           v, dym, Lpad, Dpad, dqkv, H, T, Tpad, scale, scale_log2, DropParams{},
                           nullptr);
      }
    }
    mark(h, 6, st);
    // ---- c_attn: dx = dqkv W_attn^T ; dW_attn = x^T dqkv ; db_attn = colsum(dqkv)
    (void)hipStreamWaitEvent(st, h->ev_join, 0);
    Epi2RowMajor e_dx{(bf16_t*)dx, C, nullptr};
    if (use_gemm3(M, C))
      launch_gemm3<GA_DGRAD3_TILE, true, true>(dqkv, N3, (const bf16_t*)W_attn, N3, M, C, N3,
                                               e_dx, st);
    else
      launch_gemm2<GA_DGRAD_TILE, true, true>(dqkv, N3, (const bf16_t*)W_attn, N3, M, C, N3,
                                              e_dx, st);
    Epi2PartialCS e_wa{part, N3, (size_t)(C + 1) * N3, C, db_attn ? 1 : 0};
    int s2;
    {
      constexpr int tile[] = {GA_WGRAD_ATTN_TILE};
      const int tiles = ((C + tile[0] - 1) / tile[0]) * ((N3 + tile[1] - 1) / tile[1]);
      s2 = std::max(1, std::min(kWgradSplits, 256 * GA_WGRAD_ATTN_PER_CU / tiles));
    }
    const int n2 = launch_gemm2<GA_WGRAD_ATTN_TILE, false, false>(
        (const bf16_t*)x, C, dqkv, N3, C, N3, M, e_wa, st, s2);
    // db_attn = colsum(dqkv): row C of the slices' partials, reduced with them
    hipLaunchKernelGGL(reduce_partials4_bf16_kernel, dim3(rblocks), dim3(256), 0, st, part, n2,
                       (size_t)C * N3, (size_t)(C + 1) * N3, (bf16_t*)dW_attn,
                       db_attn ? (size_t)N3 : 0, (bf16_t*)db_attn);
  } else {
    const float* qkv = (const float*)h->qkv;
    const float* o = (const float*)h->o;
    float* dym = (float*)h->dym;
    float* dqkv = (float*)h->dqkv;
    EpiRowMajor<float> e_dym{dym, C, nullptr};
    launch_gemm_f32<true, true>((const float*)dY, C, (const float*)W_proj, C, M, C, C, e_dym, st);
    EpiRowMajor<float> e_wp{(float*)dW_proj, C, nullptr};
    launch_gemm_f32<false, false>(o, C, (const float*)dY, C, C, C, M, e_wp, st);
    if (db_proj) {
      hipLaunchKernelGGL(colsum_partial_kernel<float>, dim3((C + 255) / 256, ncs), dim3(256), 0,
                         st, (const float*)dY, M, C, C, rows_per, cpart);
      hipLaunchKernelGGL(reduce_colparts_kernel<float>, dim3((C + 63) / 64), dim3(256), 0, st,
                         cpart, ncs, C, (float*)db_proj);
    }
    mark(h, 5, st);
    const dim3 dgrid((unsigned)((M * (long)H + 255) / 256));
    const dim3 tgrid((unsigned)((M * (long)H + 63) / 64));
    const float* q = qkv;
    const float* k = qkv + head_elems;
    const float* v = qkv + 2 * head_elems;
    if (hs == 64) {
      hipLaunchKernelGGL((attn_delta_kernel<64, float>), dgrid, dim3(256), 0, st, dym, o,
                         h->delta, B, H, T);
      hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<64>, tgrid, dim3(64), 0, st, q, k, v, dym,
                         h->lse, h->delta, dqkv, B, H, T, scale, scale_log2);
      hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<64>, tgrid, dim3(64), 0, st, q, k, v, dym,
                         h->lse, h->delta, dqkv, B, H, T, scale, scale_log2);
    } else {
      hipLaunchKernelGGL((attn_delta_kernel<32, float>), dgrid, dim3(256), 0, st, dym, o,
                         h->delta, B, H, T);
      hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<32>, tgrid, dim3(64), 0, st, q, k, v, dym,
                         h->lse, h->delta, dqkv, B, H, T, scale, scale_log2);
      hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<32>, tgrid, dim3(64), 0, st, q, k, v, dym,
                         h->lse, h->delta, dqkv, B, H, T, scale, scale_log2);
    }
    mark(h, 6, st);
    EpiRowMajor<float> e_dx{(float*)dx, C, nullptr};
    launch_gemm_f32<true, true>(dqkv, N3, (const float*)W_attn, N3, M, C, N3, e_dx, st);
    EpiRowMajor<float> e_wa{(float*)dW_attn, N3, nullptr};
    launch_gemm_f32<false, false>((const float*)x, C, dqkv, N3, C, N3, M, e_wa, st);
    if (db_attn) {
      hipLaunchKernelGGL(colsum_partial_kernel<float>, dim3((N3 + 255) / 256, ncs), dim3(256), 0,
                         st, dqkv, M, N3, N3, rows_per, cpart);
      hipLaunchKernelGGL(reduce_colparts_kernel<float>, dim3((N3 + 63) / 64), dim3(256), 0, st,
                         cpart, ncs, N3, (float*)db_attn);
    }
  }
  mark(h, 7, st);
  return launch_status();
}

}  // extern "C"
