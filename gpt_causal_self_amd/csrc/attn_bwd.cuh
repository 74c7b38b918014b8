// attn_bwd.cuh -- the gradient formulas of the fused causal attention, the
// fp32 backward kernels, and the small reduction kernels of the layer's
// backward (the bf16 attention kernels are in attn_bwd2.cuh).
//
// Given the forward's q, k, v (head-major), its merged output o, the softmax
// log-sum-exp L_i of every row and the upstream gradient dO of the merged
// heads, the exact gradient of o_i = sum_{j<=i} p_ij v_j,
// p_ij = exp(s_ij - L_i), s_ij = q_i.k_j / sqrt(hs) is
//   D_i   = sum_d dO_id o_id                (= sum_j p_ij dP_ij)
//   dP_ij = dO_i . v_j
//   dS_ij = p_ij (dP_ij - D_i)
//   dv_j  = sum_{i>=j} p_ij dO_i
//   dk_j  = (1/sqrt(hs)) sum_{i>=j} dS_ij q_i
//   dq_i  = (1/sqrt(hs)) sum_{j<=i} dS_ij k_j
// (the chain rule through the forward on page "nanoGPT global flow
// walkthrough", section 2.5 (B), steps 3-7).  P is recomputed from L, never
// stored.  dq is produced by its own kernel and dk, dv by another, so every
// output element is written by exactly one thread: no atomics,
// deterministic results.
//
// The gradients land in dqkv [B][T][3C] (columns: q block, k block, v block;
// head h at h*hs within each), the layout the c_attn backward GEMMs read.
//
// With dropout on the weights (DROP; philox.cuh) o_i = sum_j p_ij z_ij v_j,
// z_ij = 1/(1-p) for kept and 0 for dropped weights: dv_j sums p_ij z_ij dO_i,
// dP_ij = z_ij dO_i . v_j, and D_i = dO_i . o_i is unchanged.
#pragma once

#include "common.cuh"
#include "gemm.cuh"
#include "philox.cuh"

namespace gpt_attn {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ delta
// D[bh][t] = sum_d dO[b][t][h*HS + d] * O[b][t][h*HS + d]; one thread per
// (b, t, h) (fp32 element type).
template <int HS, class T_>
__global__ __launch_bounds__(256) void attn_delta_kernel(const T_* __restrict__ dO,
                                                         const T_* __restrict__ O,
                                                         float* __restrict__ D, int B,
                                                         int H, int T) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)B * T * H) return;
  const int h = (int)(idx % H);
  const long bt = idx / H;
  const int t = (int)(bt % T), b = (int)(bt / T);
  const size_t off = (size_t)bt * H * HS + (size_t)h * HS;
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < HS; ++d) s = fmaf(load1(dO + off + d), load1(O + off + d), s);
  D[((size_t)b * H + h) * T + t] = s;
}

// Sum over 4 (Q = 4) or 8 (Q = 8) consecutive lanes with DPP moves (quad
// swaps, then the mirrored lane of the half-row); every lane of the group
// ends with the group's total.
template <int Q>
__device__ __forceinline__ float lane_group_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if (Q == 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

// ------------------------------------------------------ output dropout
// dYd[m][n] = dY[m][n] * z_mn (z = 1/(1-p) kept, 0 dropped; the c_proj
// output mask of philox.cuh), one thread per 4 columns.
__global__ __launch_bounds__(256) void dropout_grad_kernel(const bf16_t* __restrict__ dY,
                                                           bf16_t* __restrict__ dYd, long M,
                                                           int C, DropParams drop) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;  // group of 4 columns
  const int per = C / 4;
  if (i >= M * per) return;
  const long m = i / per;
  const int n = (int)(i - m * per) * 4;
  const uint4 w =
      philox4x32_10(make_uint4((uint32_t)n >> 2, (uint32_t)m, 0u, 2u), drop.k0, drop.k1);
  const uint2 u = *reinterpret_cast<const uint2*>(dY + m * C + n);
  const float z0 = w.x >= drop.thresh ? drop.scale : 0.f;
  const float z1 = w.y >= drop.thresh ? drop.scale : 0.f;
  const float z2 = w.z >= drop.thresh ? drop.scale : 0.f;
  const float z3 = w.w >= drop.thresh ? drop.scale : 0.f;
  uint2 o;
  o.x = pack_bf16x2(bf2f(u.x & 0xffff) * z0, bf2f(u.x >> 16) * z1);
  o.y = pack_bf16x2(bf2f(u.y & 0xffff) * z2, bf2f(u.y >> 16) * z3);
  *reinterpret_cast<uint2*>(dYd + m * C + n) = o;
}

// ================================================================== fp32
// Straightforward kernels for the fp32 element type: one thread per key
// (dk, dv) or per query (dq), looping over the visible partners.
template <int HS>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(
    const float* __restrict__ Qg, const float* __restrict__ Kg, const float* __restrict__ Vg,
    const float* __restrict__ dOg, const float* __restrict__ lse, const float* __restrict__ Dg,
    float* __restrict__ dqkv, int B, int H, int T, float scale, float scale_log2) {
  const long idx = (long)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (long)B * H * T) return;
  const int j = (int)(idx % T);
  const int bh = (int)(idx / T);
  const int b = bh / H, h = bh - b * H;
  const int C = H * HS;
  const size_t head = (size_t)bh * T * HS;
  float k[HS], v[HS], dk[HS], dv[HS];
#pragma unroll
  for (int d = 0; d < HS; ++d) {
    k[d] = Kg[head + (size_t)j * HS + d];
    v[d] = Vg[head + (size_t)j * HS + d];
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  for (int i = j; i < T; ++i) {
    const float* q = Qg + head + (size_t)i * HS;
    const float* g = dOg + ((size_t)b * T + i) * C + (size_t)h * HS;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < HS; ++d) {
      s = fmaf(q[d], k[d], s);
      dp = fmaf(g[d], v[d], dp);
    }
    const float p = __builtin_amdgcn_exp2f(s * scale_log2 - lse[(size_t)bh * T + i] * kLog2e);
    const float ds = p * (dp - Dg[(size_t)bh * T + i]);
#pragma unroll
    for (int d = 0; d < HS; ++d) {
      dk[d] = fmaf(ds, q[d], dk[d]);
      dv[d] = fmaf(p, g[d], dv[d]);
    }
  }
  float* row = dqkv + ((size_t)b * T + j) * 3 * C + (size_t)h * HS;
#pragma unroll
  for (int d = 0; d < HS; ++d) {
    row[C + d] = dk[d] * scale;
    row[2 * C + d] = dv[d];
  }
}

template <int HS>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(
    const float* __restrict__ Qg, const float* __restrict__ Kg, const float* __restrict__ Vg,
    const float* __restrict__ dOg, const float* __restrict__ lse, const float* __restrict__ Dg,
    float* __restrict__ dqkv, int B, int H, int T, float scale, float scale_log2) {
  const long idx = (long)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (long)B * H * T) return;
  const int i = (int)(idx % T);
  const int bh = (int)(idx / T);
  const int b = bh / H, h = bh - b * H;
  const int C = H * HS;
  const size_t head = (size_t)bh * T * HS;
  float q[HS], g[HS], dq[HS];
#pragma unroll
  for (int d = 0; d < HS; ++d) {
    q[d] = Qg[head + (size_t)i * HS + d];
    g[d] = dOg[((size_t)b * T + i) * C + (size_t)h * HS + d];
    dq[d] = 0.f;
  }
  const float L2 = lse[(size_t)bh * T + i] * kLog2e;
  const float Di = Dg[(size_t)bh * T + i];
  for (int j = 0; j <= i; ++j) {
    const float* k = Kg + head + (size_t)j * HS;
    const float* v = Vg + head + (size_t)j * HS;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < HS; ++d) {
      s = fmaf(q[d], k[d], s);
      dp = fmaf(g[d], v[d], dp);
    }
    const float ds = __builtin_amdgcn_exp2f(s * scale_log2 - L2) * (dp - Di);
#pragma unroll
    for (int d = 0; d < HS; ++d) dq[d] = fmaf(ds, k[d], dq[d]);
  }
  float* row = dqkv + ((size_t)b * T + i) * 3 * C + (size_t)h * HS;
#pragma unroll
  for (int d = 0; d < HS; ++d) row[d] = dq[d] * scale;
}

// ============================================================ reductions
// Column sums of X [M][N] (row stride ld) over the row range of split
// blockIdx.y: part[split][n] (fp32).  One thread per column.
template <class T_>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T_* __restrict__ X, int M,
                                                             int N, int ld, int rows_per_split,
                                                             float* __restrict__ part) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int r0 = blockIdx.y * rows_per_split;
  const int r1 = min(M, r0 + rows_per_split);
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += load1(X + (size_t)r * ld + n);
  part[(size_t)blockIdx.y * N + n] = s;
}

// out[i] = sum_{s < S} part[s*stride + i] for i < n, in the output type.
// out[i..i+3] = sum_k part[k][i..i+3] (n, n2, stride multiples of 4; 16-byte
// partial loads).  The n2 elements after the first n of each slice (a
// weight gradient's bias row) go to out2 in the same pass.
__global__ __launch_bounds__(256) void reduce_partials4_bf16_kernel(
    const float* __restrict__ part, int S, size_t n, size_t stride, bf16_t* __restrict__ out,
    size_t n2, bf16_t* __restrict__ out2) {
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n + n2;
       i += (size_t)gridDim.x * 256 * 4) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < S; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(part + (size_t)k * stride + i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    uint2 w;
    w.x = pack_bf16x2(s.x, s.y);
    w.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<uint2*>(i < n ? out + i : out2 + (i - n)) = w;
  }
}

template <class T_>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part,
                                                              int S, size_t n, size_t stride,
                                                              T_* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (size_t)gridDim.x * 256) {
    float s = 0.f;
    for (int k = 0; k < S; ++k) s += part[(size_t)k * stride + i];
    store1(out + i, s);
  }
}

// Column sums of S partial rows: out[c] = sum_k part[k * N + c].  One block
// per 64 columns; its 4 waves split the partial rows (coalesced across the
// 64 columns) and combine through LDS, so even N = 768 spreads over 12
// blocks and no thread walks all S rows.
template <class T_>
__global__ __launch_bounds__(256) void reduce_colparts_kernel(const float* __restrict__ part,
                                                              int S, int N,
                                                              T_* __restrict__ out) {
  __shared__ float red[4][64];
  const int tid = threadIdx.x, c = tid & 63, sl = tid >> 6;
  const int col = blockIdx.x * 64 + c;
  float s = 0.f;
  if (col < N) {
#pragma unroll 4
    for (int k = sl; k < S; k += 4) s += part[(size_t)k * N + col];
  }
  red[sl][c] = s;
  __syncthreads();
  if (sl == 0 && col < N) store1(out + col, (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]));
}

}  // namespace gpt_attn
