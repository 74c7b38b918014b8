// layernorm.cuh -- row LayerNorm of bf16 activations (the ln_1 / ln_2 of a
// Pre-LN Block).
//
//   out[m][c] = (x[m][c] - mu_m) / sqrt(var_m + 1e-5) * w[c] + b[c]
//
// mu_m and the biased variance var_m over the C features of row m, as
// F.layer_norm (page "nanoGPT global flow walkthrough", section 2.5 (A)).
// L lanes per row (a half wave for rows of up to 768 features, so that no
// lane idles; a whole wave for longer rows): each lane holds up to CH
// 16-byte chunks (8 features) of the row in registers, all of them loaded
// before the first is used, so x is read once with every load of a lane in
// flight together.  The mean and then the centred sum of squares are fp32
// reductions over the L lanes (two passes over registers, no cancellation
// from E[x^2] - mu^2).  The kernel is HBM-bound: 2 bytes read and 2 written
// per feature (plus w and b, cache resident).
#pragma once

#include "common.cuh"

namespace gpt_attn {

template <int L>
__device__ __forceinline__ float ln_lane_sum(float v) {
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int L, int CH>
__global__ __launch_bounds__(256) void layernorm_bf16_kernel(const bf16_t* __restrict__ x,
                                                             const bf16_t* __restrict__ w,
                                                             const bf16_t* __restrict__ b,
                                                             bf16_t* __restrict__ out, int M,
                                                             int C) {
  static_assert(L == 32 || L == 64, "a row is held by a half wave or a wave");
  const int gl = threadIdx.x % L;
  const int row = blockIdx.x * (256 / L) + threadIdx.x / L;
  // both halves of a wave take part in the shuffles, so a half wave past the
  // last row still runs the reductions (on zeros) and only skips the stores
  const bool live = row < M;
  const int nch = C >> 3;
  const bf16_t* xr = x + (size_t)(live ? row : 0) * C;
  // weight and bias chunks: they do not depend on the statistics, so rows of
  // up to 4 chunks per lane load them up front (longer rows load them at the
  // end, to keep the registers for the row itself)
  constexpr bool kEarly = CH <= 4;
  auto load_wb = [&](int k, uint4& wk, uint4& bk) {
    const int c = gl + L * k;
    wk = c < nch ? *reinterpret_cast<const uint4*>(w + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    bk = (b && c < nch) ? *reinterpret_cast<const uint4*>(b + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 xv[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int c = gl + L * k;
    xv[k] = (live && c < nch) ? *reinterpret_cast<const uint4*>(xr + 8 * c)
                              : make_uint4(0u, 0u, 0u, 0u);
  }
  uint4 wv[kEarly ? CH : 1], bv[kEarly ? CH : 1];
  if constexpr (kEarly) {
#pragma unroll
    for (int k = 0; k < CH; ++k) load_wb(k, wv[k], bv[k]);
  }
  // chunks past the row are zeros: they add nothing to the sum
  float v[CH][8];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const unsigned wd[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[k][2 * e] = bf2f(wd[e] & 0xffff);
      v[k][2 * e + 1] = bf2f(wd[e] >> 16);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[k][e];
  }
  const float mean = ln_lane_sum<L>(s) / (float)C;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    if (gl + L * k < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[k][e] - mean;
        q += d * d;
      }
    }
  }
  const float rstd = 1.f / sqrtf(ln_lane_sum<L>(q) / (float)C + 1e-5f);
  if (!live) return;
  bf16_t* orow = out + (size_t)row * C;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int c = gl + L * k;
    if (c < nch) {
      uint4 wk, bk;
      if constexpr (kEarly) {
        wk = wv[k];
        bk = bv[k];
      } else {
        load_wb(k, wk, bk);
      }
      const unsigned ww[4] = {wk.x, wk.y, wk.z, wk.w};
      const unsigned bb[4] = {bk.x, bk.y, bk.z, bk.w};
      unsigned o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y0 = (v[k][2 * e] - mean) * rstd * bf2f(ww[e] & 0xffff) + bf2f(bb[e] & 0xffff);
        const float y1 = (v[k][2 * e + 1] - mean) * rstd * bf2f(ww[e] >> 16) + bf2f(bb[e] >> 16);
        o[e] = pack_bf16x2(y0, y1);
      }
      *reinterpret_cast<uint4*>(orow + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// Launch over M rows; C % 8 == 0, C <= 8192.
template <int L, int CH>
inline void launch_layernorm_as(const bf16_t* x, const bf16_t* w, const bf16_t* b, bf16_t* out,
                                int M, int C, hipStream_t st) {
  constexpr int rows = 256 / L;
  hipLaunchKernelGGL((layernorm_bf16_kernel<L, CH>), dim3((M + rows - 1) / rows), dim3(256), 0,
                     st, x, w, b, out, M, C);
}

inline void launch_layernorm(const bf16_t* x, const bf16_t* w, const bf16_t* b, bf16_t* out,
                             int M, int C, hipStream_t st) {
  const int nch = C / 8;
  if (nch <= 32)
    launch_layernorm_as<32, 1>(x, w, b, out, M, C, st);
  else if (nch <= 64)
    launch_layernorm_as<32, 2>(x, w, b, out, M, C, st);
  else if (nch <= 96)
    launch_layernorm_as<32, 3>(x, w, b, out, M, C, st);
  else if (nch <= 128)
    launch_layernorm_as<64, 2>(x, w, b, out, M, C, st);
  else if (nch <= 256)
    launch_layernorm_as<64, 4>(x, w, b, out, M, C, st);
  else
    launch_layernorm_as<64, 16>(x, w, b, out, M, C, st);
}

}  // namespace gpt_attn
