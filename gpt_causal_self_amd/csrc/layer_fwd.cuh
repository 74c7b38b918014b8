// layer_fwd.cuh -- launch sequence of the bf16 layer forward, shared by
// gpt_attn_forward and the Pre-LN block entry point.
#pragma once

#include "attn_fwd.cuh"
#include "gemm2.cuh"
#include "handle.cuh"

namespace gpt_attn {

// c_proj epilogue with the Block's residual: out = acc + bias + res, one
// rounding (page "nanoGPT global flow walkthrough", section 2.5: the attention
// output is added back onto x).  Stored straight from the accumulators.
struct Epi2RowMajorRes {
  bf16_t* out;
  int ldc;
  const bf16_t* bias;  // may be NULL
  const bf16_t* res;   // [M][ldc]
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      const uint2 u = *reinterpret_cast<const uint2*>(bias + n);
      b[0] = bf2f(u.x & 0xffff); b[1] = bf2f(u.x >> 16);
      b[2] = bf2f(u.y & 0xffff); b[3] = bf2f(u.y >> 16);
    }
    const uint2 r = *reinterpret_cast<const uint2*>(res + (size_t)m * ldc + n);
    uint2 w;
    w.x = pack_bf16x2(v[0] + b[0] + bf2f(r.x & 0xffff), v[1] + b[1] + bf2f(r.x >> 16));
    w.y = pack_bf16x2(v[2] + b[2] + bf2f(r.y & 0xffff), v[3] + b[3] + bf2f(r.y >> 16));
    *reinterpret_cast<uint2*>(out + (size_t)m * ldc + n) = w;
  }
};

// c_proj epilogue with dropout on the c_proj output (philox.cuh) and an
// optional residual: out = res + keep * (acc + bias) / (1 - p), one rounding.
struct Epi2RowMajorDrop {
  bf16_t* out;
  int ldc;
  const bf16_t* bias;  // may be NULL
  const bf16_t* res;   // may be NULL
  DropParams drop;
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      const uint2 u = *reinterpret_cast<const uint2*>(bias + n);
      b[0] = bf2f(u.x & 0xffff); b[1] = bf2f(u.x >> 16);
      b[2] = bf2f(u.y & 0xffff); b[3] = bf2f(u.y >> 16);
    }
    float r[4] = {0.f, 0.f, 0.f, 0.f};
    if (res) {
      const uint2 u = *reinterpret_cast<const uint2*>(res + (size_t)m * ldc + n);
      r[0] = bf2f(u.x & 0xffff); r[1] = bf2f(u.x >> 16);
      r[2] = bf2f(u.y & 0xffff); r[3] = bf2f(u.y >> 16);
    }
    // columns n..n+3 (n % 4 == 0): one Philox call
    const uint4 w = philox4x32_10(make_uint4((uint32_t)n >> 2, (uint32_t)m, 0u, 2u), drop.k0,
                                  drop.k1);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = r[e] + (wd[e] >= drop.thresh ? (v[e] + b[e]) * drop.scale : 0.f);
    uint2 st;
    st.x = pack_bf16x2(o[0], o[1]);
    st.y = pack_bf16x2(o[2], o[3]);
    *reinterpret_cast<uint2*>(out + (size_t)m * ldc + n) = st;
  }
};

// c_attn GEMM -> fused causal attention -> c_proj GEMM on stream st.
// residual == NULL: y = layer(x); else y = residual + layer(x).
// lse != NULL: also store the softmax log-sum-exp rows for the backward.
// drop != NULL: dropout on the attention weights and the c_proj output.
inline void layer_forward_bf16(const gpt_attn_handle* h, const bf16_t* x, int B, int T,
                               const bf16_t* W_attn, const bf16_t* b_attn,
                               const bf16_t* W_proj, const bf16_t* b_proj, bf16_t* y,
                               const bf16_t* residual, float* lse, hipStream_t st,
                               const DropParams* drop = nullptr) {
  const int C = h->C, H = h->H, hs = h->hs;
  const int M = B * T;
  const size_t head_elems = (size_t)B * H * T * hs;  // one of q, k, v
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hs));
  bf16_t* qkv = (bf16_t*)h->qkv;
  bf16_t* o = (bf16_t*)h->o;
  Epi2QKV e1{qkv, b_attn, B, T, C, H, hs};
  mark(h, 0, st);
  launch_gemm2<GA_QKV_TILE, true, false>(x, C, W_attn, 3 * C, M, 3 * C, C, e1, st);
  mark(h, 1, st);
  const dim3 agrid(B * H, (T + kAttnBQ - 1) / kAttnBQ);
  if (drop) {
    if (hs == 64)
      hipLaunchKernelGGL((attn_fwd2_bf16_kernel<64, GA_ATTN_STAGES, true>), agrid, dim3(256), 0,
                         st, qkv, qkv + head_elems, qkv + 2 * head_elems, o, lse, H, T,
                         scale_log2, *drop);
    else
      hipLaunchKernelGGL((attn_fwd2_bf16_kernel<32, GA_ATTN_STAGES, true>), agrid, dim3(256), 0,
                         st, qkv, qkv + head_elems, qkv + 2 * head_elems, o, lse, H, T,
                         scale_log2, *drop);
  } else if (hs == 64) {
    hipLaunchKernelGGL((attn_fwd2_bf16_kernel<64, GA_ATTN_STAGES>), agrid, dim3(256), 0, st,
                       qkv, qkv + head_elems, qkv + 2 * head_elems, o, lse, H, T, scale_log2,
                       DropParams{});
  } else {
    hipLaunchKernelGGL((attn_fwd2_bf16_kernel<32, GA_ATTN_STAGES>), agrid, dim3(256), 0, st,
                       qkv, qkv + head_elems, qkv + 2 * head_elems, o, lse, H, T, scale_log2,
                       DropParams{});
  }
  mark(h, 2, st);
  if (drop) {
    Epi2RowMajorDrop e3{y, C, b_proj, residual, *drop};
    launch_gemm2<GA_PROJ_TILE, true, false>(o, C, W_proj, C, M, C, C, e3, st);
  } else if (residual) {
    Epi2RowMajorRes e3{y, C, b_proj, residual};
    launch_gemm2<GA_PROJ_TILE, true, false>(o, C, W_proj, C, M, C, C, e3, st);
  } else {
    Epi2RowMajor e3{y, C, b_proj};
    launch_gemm2<GA_PROJ_TILE, true, false>(o, C, W_proj, C, M, C, C, e3, st);
  }
  mark(h, 3, st);
}

}  // namespace gpt_attn
