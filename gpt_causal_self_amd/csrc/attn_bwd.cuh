// attn_bwd.cuh -- backward of the fused causal attention, plus the small
// reduction kernels of the layer's backward.
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
// stored.  dq is produced by its own kernel (one block per query tile) and
// dk, dv by another (one block per key tile), so every output element is
// written by exactly one wave: no atomics, deterministic results.
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
// (b, t, h).
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

// D[bh][t] = dO[b][t][h*HS..] . O[b][t][h*HS..] for bf16: a thread takes 8
// consecutive elements of a row (16-byte loads of both tensors), the HS/8
// threads of one head meet with lane_group_sum.
template <int HS>
__global__ __launch_bounds__(256) void attn_delta_bf16_kernel(const bf16_t* __restrict__ dO,
                                                              const bf16_t* __restrict__ O,
                                                              float* __restrict__ D, int B, int H,
                                                              int T) {
  constexpr int Q = HS / 8;
  const int C = H * HS, per = C / 8;
  const long g = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)B * T * per;
  const bool ok = g < total;
  float s = 0.f;
  long row = 0;
  int c = 0;
  if (ok) {
    row = g / per;
    c = (int)(g - row * per);
    const uint4 a = *reinterpret_cast<const uint4*>(dO + row * C + 8 * c);
    const uint4 o = *reinterpret_cast<const uint4*>(O + row * C + 8 * c);
    const unsigned wa[4] = {a.x, a.y, a.z, a.w}, wo[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(bf2f(wa[e] & 0xffff), bf2f(wo[e] & 0xffff), s);
      s = fmaf(bf2f(wa[e] >> 16), bf2f(wo[e] >> 16), s);
    }
  }
  s = lane_group_sum<Q>(s);  // every lane takes part (groups never straddle the end)
  if (ok && c % Q == 0) {
    const int h = c / Q;
    const long b = row / T, t = row - b * T;
    D[((size_t)b * H + h) * T + t] = s;
  }
}

// Column sums of a bf16 matrix: block (x, y) sums columns [64x, 64x + 64)
// over rows [y * rows_per, (y + 1) * rows_per); 256 threads = 8 column groups
// (16-byte loads of 8 columns) x 32 row slots, the slot sums meet in LDS in a
// fixed order; part[y][n] receives the block's sums.  N % 8 == 0.
__global__ __launch_bounds__(256) void colsum_bf16_kernel(const bf16_t* __restrict__ X, int M,
                                                          int N, int ld, int rows_per,
                                                          float* __restrict__ part) {
  __shared__ float red[32][64];
  const int tid = threadIdx.x, cg = tid & 7, slot = tid >> 3;
  const int n = blockIdx.x * 64 + 8 * cg;
  const int r0 = blockIdx.y * rows_per, r1 = min(M, r0 + rows_per);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (n < N) {
    for (int r = r0 + slot; r < r1; r += 32 * 4) {
      uint4 u[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        u[q] = r + 32 * q < r1 ? *reinterpret_cast<const uint4*>(X + (size_t)(r + 32 * q) * ld + n)
                               : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const unsigned w[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf2f(w[e] & 0xffff);
          acc[2 * e + 1] += bf2f(w[e] >> 16);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[slot][8 * cg + e] = acc[e];
  __syncthreads();
  if (tid < 64 && blockIdx.x * 64 + tid < N) {
    float t = 0.f;
    for (int sl = 0; sl < 32; ++sl) t += red[sl][tid];
    part[(size_t)blockIdx.y * N + blockIdx.x * 64 + tid] = t;
  }
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

// ========================================================= bf16, dK / dV
// One block = 4 waves = 128 keys of one (b, h); wave w owns 32 keys and
// keeps them (as MFMA B operands) in registers.  The block walks the query
// tiles of 64 that can see its keys.  Per query tile a wave computes
//   S   = Q K^T  and  dP = dO V^T   (queries on MFMA rows, its keys on
//                                    columns: lane = key)
//   P   = exp2(S*scale*log2e - L_i*log2e) (masked), dS = P (dP - D_i)
//   dV^T += dO^T P ,  dK^T += Q^T dS  (d on rows, keys on columns)
// The probability / dS registers are already the B operands of the last two
// products (queries as the k index, in the accumulator's order); dO^T and
// Q^T come from transposed LDS copies read in that same order.
constexpr int kBwdBK = 128;  // keys per block (dK/dV kernel)
constexpr int kBwdBQ = 64;   // queries per tile (dK/dV kernel)

template <int HS, bool DROP = false>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_bf16_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg,
    const bf16_t* __restrict__ Vg, const bf16_t* __restrict__ dOg,
    const float* __restrict__ lse, const float* __restrict__ Dg, bf16_t* __restrict__ dqkv,
    int H, int T, float scale, float scale_log2, DropParams drop = {}) {
  constexpr int P1 = HS + 8;       // [q][d] pitch
  constexpr int P2 = kBwdBQ + 4;   // [d][q] pitch
  __shared__ __align__(16) bf16_t Qs[kBwdBQ * P1];
  __shared__ __align__(16) bf16_t dOs[kBwdBQ * P1];
  __shared__ __align__(16) bf16_t Qt[HS * P2];
  __shared__ __align__(16) bf16_t dOt[HS * P2];
  __shared__ float Ls[kBwdBQ];
  __shared__ float Ds[kBwdBQ];

  const int nkt = (T + kBwdBK - 1) / kBwdBK;
  const int bh = blockIdx.x;
  const int kt = nkt - 1 - (int)blockIdx.y;  // blocks with few query tiles last
  const int b = bh / H, h = bh - b * H;
  const int C = H * HS;
  const size_t head = (size_t)bh * T * HS;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hi = lane >> 5;
  const int kb0 = kt * kBwdBK;
  const int kw0 = kb0 + wid * 32;
  const int mykey = kw0 + (lane & 31);

  // this wave's keys and values as B operands: lane holds row mykey, dims
  // 16*kk + 8*hi + 0..7
  bf16x8 kf[HS / 16], vf[HS / 16];
#pragma unroll
  for (int kk = 0; kk < HS / 16; ++kk) {
    if (mykey < T) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(Kg + head + (size_t)mykey * HS + 16 * kk + 8 * hi);
      vf[kk] = *reinterpret_cast<const bf16x8*>(Vg + head + (size_t)mykey * HS + 16 * kk + 8 * hi);
    } else {
      kf[kk] = bf16x8{};
      vf[kk] = bf16x8{};
    }
  }
  floatx16 dk[HS / 32], dv[HS / 32];
#pragma unroll
  for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  const bf16_t* dOb = dOg + (size_t)b * T * C + (size_t)h * HS;  // row stride C
  for (int i0 = kb0; i0 < T; i0 += kBwdBQ) {
    // ---- stage Q, dO (both orientations), L and D of queries i0 .. i0+63
    constexpr int CH = kBwdBQ * HS / 8;
    for (int c = tid; c < CH; c += 256) {
      const int q = c / (HS / 8), dc = c % (HS / 8);
      uint4 a = make_uint4(0, 0, 0, 0), g = make_uint4(0, 0, 0, 0);
      if (i0 + q < T) {
        a = *reinterpret_cast<const uint4*>(Qg + head + (size_t)(i0 + q) * HS + dc * 8);
        g = *reinterpret_cast<const uint4*>(dOb + (size_t)(i0 + q) * C + dc * 8);
      }
      *reinterpret_cast<uint4*>(&Qs[q * P1 + dc * 8]) = a;
      *reinterpret_cast<uint4*>(&dOs[q * P1 + dc * 8]) = g;
    }
    constexpr int TB = (kBwdBQ / 4) * (HS / 4);  // 4 x 4 transposition blocks
    for (int t4 = tid; t4 < TB; t4 += 256) {
      const int dg = t4 % (HS / 4), qg = t4 / (HS / 4);
      uint2 a[4], g[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int q = i0 + qg * 4 + kk;
        if (q < T) {
          a[kk] = *reinterpret_cast<const uint2*>(Qg + head + (size_t)q * HS + dg * 4);
          g[kk] = *reinterpret_cast<const uint2*>(dOb + (size_t)q * C + dg * 4);
        } else {
          a[kk] = make_uint2(0, 0);
          g[kk] = make_uint2(0, 0);
        }
      }
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const int sh = (dd & 1) * 16;
        uint2 oa, og;
        oa.x = (((dd < 2 ? a[0].x : a[0].y) >> sh) & 0xffffu) |
               ((((dd < 2 ? a[1].x : a[1].y) >> sh) & 0xffffu) << 16);
        oa.y = (((dd < 2 ? a[2].x : a[2].y) >> sh) & 0xffffu) |
               ((((dd < 2 ? a[3].x : a[3].y) >> sh) & 0xffffu) << 16);
        og.x = (((dd < 2 ? g[0].x : g[0].y) >> sh) & 0xffffu) |
               ((((dd < 2 ? g[1].x : g[1].y) >> sh) & 0xffffu) << 16);
        og.y = (((dd < 2 ? g[2].x : g[2].y) >> sh) & 0xffffu) |
               ((((dd < 2 ? g[3].x : g[3].y) >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint2*>(&Qt[(dg * 4 + dd) * P2 + qg * 4]) = oa;
        *reinterpret_cast<uint2*>(&dOt[(dg * 4 + dd) * P2 + qg * 4]) = og;
      }
    }
    if (tid < kBwdBQ) {
      const int q = i0 + tid;
      Ls[tid] = q < T ? lse[(size_t)bh * T + q] * kLog2e : 0.f;
      Ds[tid] = q < T ? Dg[(size_t)bh * T + q] : 0.f;
    }
    __syncthreads();

    if (i0 + kBwdBQ - 1 >= kw0) {  // some query of the tile sees a key of the wave
      floatx16 s[2], dp[2];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[qh][r] = 0.f;
          dp[qh][r] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < HS / 16; ++kk) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(
              &Qs[(qh * 32 + (lane & 31)) * P1 + 16 * kk + 8 * hi]);
          const bf16x8 ga = *reinterpret_cast<const bf16x8*>(
              &dOs[(qh * 32 + (lane & 31)) * P1 + 16 * kk + 8 * hi]);
          s[qh] = mfma32(qa, kf[kk], s[qh]);
          dp[qh] = mfma32(ga, vf[kk], dp[qh]);
        }
        // P and dS; lane = key mykey, register r = query qh*32 + 8(r/4) + 4hi + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qh * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const int q = i0 + ql;
          float p = __builtin_amdgcn_exp2f(s[qh][r] * scale_log2 - Ls[ql]);
          if (mykey > q || q >= T) p = 0.f;
          if constexpr (DROP) {
            // weight (query q, key mykey): word mykey % 4 of counter
            // (mykey / 4, q, bh, 1)
            const uint4 w = philox4x32_10(
                make_uint4((uint32_t)mykey >> 2, (uint32_t)q, (uint32_t)bh, 1u), drop.k0,
                drop.k1);
            const uint32_t k = mykey & 3;
            const uint32_t wd = k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
            const float z = wd >= drop.thresh ? drop.scale : 0.f;
            s[qh][r] = p * z;
            dp[qh][r] = p * (dp[qh][r] * z - Ds[ql]);
          } else {
            s[qh][r] = p;
            dp[qh][r] = p * (dp[qh][r] - Ds[ql]);
          }
        }
      }
      // dV^T += dO^T P ;  dK^T += Q^T dS   (k index = queries, permuted order)
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8 pf, sf;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pf[e] = (__bf16)s[qh][8 * u + e];
            sf[e] = (__bf16)dp[qh][8 * u + e];
          }
          const int qb = qh * 32 + 16 * u + 4 * hi;
#pragma unroll
          for (int dt = 0; dt < HS / 32; ++dt) {
            const int drow = (dt * 32 + (lane & 31)) * P2 + qb;
            uint4 w;
            uint2 lo = *reinterpret_cast<const uint2*>(&dOt[drow]);
            uint2 up = *reinterpret_cast<const uint2*>(&dOt[drow + 8]);
            w.x = lo.x; w.y = lo.y; w.z = up.x; w.w = up.y;
            dv[dt] = mfma32(__builtin_bit_cast(bf16x8, w), pf, dv[dt]);
            lo = *reinterpret_cast<const uint2*>(&Qt[drow]);
            up = *reinterpret_cast<const uint2*>(&Qt[drow + 8]);
            w.x = lo.x; w.y = lo.y; w.z = up.x; w.w = up.y;
            dk[dt] = mfma32(__builtin_bit_cast(bf16x8, w), sf, dk[dt]);
          }
        }
    }
    __syncthreads();
  }

  // ---- write dk (scaled) and dv into dqkv[b][key][C + h*HS + d], [2C + ...]
  if (mykey < T) {
    bf16_t* row = dqkv + ((size_t)b * T + mykey) * 3 * C + (size_t)h * HS;
#pragma unroll
    for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        uint2 wk, wv;
        wk.x = pack_bf16x2(dk[dt][4 * g] * scale, dk[dt][4 * g + 1] * scale);
        wk.y = pack_bf16x2(dk[dt][4 * g + 2] * scale, dk[dt][4 * g + 3] * scale);
        wv.x = pack_bf16x2(dv[dt][4 * g], dv[dt][4 * g + 1]);
        wv.y = pack_bf16x2(dv[dt][4 * g + 2], dv[dt][4 * g + 3]);
        *reinterpret_cast<uint2*>(row + C + d0) = wk;
        *reinterpret_cast<uint2*>(row + 2 * C + d0) = wv;
      }
  }
}

// ============================================================ bf16, dQ
// One block = 4 waves = 128 queries of one (b, h), like the forward: each
// wave keeps its 32 queries' q and dO rows as MFMA B operands and walks the
// key tiles of 64 at or below the diagonal:
//   S^T = K Q^T, dP^T = V dO^T (keys on rows, lane = query),
//   P^T = exp2(S^T*scale*log2e - L*log2e), dS^T = P^T (dP^T - D),
//   dQ^T += K^T dS^T.
template <int HS, bool DROP = false>
__global__ __launch_bounds__(256) void attn_bwd_dq_bf16_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg,
    const bf16_t* __restrict__ Vg, const bf16_t* __restrict__ dOg,
    const float* __restrict__ lse, const float* __restrict__ Dg, bf16_t* __restrict__ dqkv,
    int H, int T, float scale, float scale_log2, DropParams drop = {}) {
  constexpr int BQ = 128, BK = 64;
  constexpr int P1 = HS + 8;   // [key][d] pitch
  constexpr int P2 = BK + 4;   // [d][key] pitch
  __shared__ __align__(16) bf16_t Ks[BK * P1];
  __shared__ __align__(16) bf16_t Vs[BK * P1];
  __shared__ __align__(16) bf16_t Kt[HS * P2];

  const int nqt = (T + BQ - 1) / BQ;
  const int bh = blockIdx.x;
  const int qt = nqt - 1 - (int)blockIdx.y;  // heavy tiles first
  const int b = bh / H, h = bh - b * H;
  const int C = H * HS;
  const size_t head = (size_t)bh * T * HS;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hi = lane >> 5;
  const int q0 = qt * BQ + wid * 32;
  const int myq = q0 + (lane & 31);
  const bf16_t* dOb = dOg + (size_t)b * T * C + (size_t)h * HS;

  bf16x8 qf[HS / 16], gf[HS / 16];
#pragma unroll
  for (int kk = 0; kk < HS / 16; ++kk) {
    if (myq < T) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(Qg + head + (size_t)myq * HS + 16 * kk + 8 * hi);
      gf[kk] = *reinterpret_cast<const bf16x8*>(dOb + (size_t)myq * C + 16 * kk + 8 * hi);
    } else {
      qf[kk] = bf16x8{};
      gf[kk] = bf16x8{};
    }
  }
  const float L2 = myq < T ? lse[(size_t)bh * T + myq] * kLog2e : 0.f;
  const float Dq = myq < T ? Dg[(size_t)bh * T + myq] : 0.f;
  floatx16 dq[HS / 32];
#pragma unroll
  for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  const int kv_end = min(T, (qt + 1) * BQ);
  for (int j0 = 0; j0 < kv_end; j0 += BK) {
    constexpr int CH = BK * HS / 8;
    for (int c = tid; c < CH; c += 256) {
      const int key = c / (HS / 8), dc = c % (HS / 8);
      uint4 a = make_uint4(0, 0, 0, 0), v = make_uint4(0, 0, 0, 0);
      if (j0 + key < T) {
        a = *reinterpret_cast<const uint4*>(Kg + head + (size_t)(j0 + key) * HS + dc * 8);
        v = *reinterpret_cast<const uint4*>(Vg + head + (size_t)(j0 + key) * HS + dc * 8);
      }
      *reinterpret_cast<uint4*>(&Ks[key * P1 + dc * 8]) = a;
      *reinterpret_cast<uint4*>(&Vs[key * P1 + dc * 8]) = v;
    }
    constexpr int TB = (BK / 4) * (HS / 4);
    for (int t4 = tid; t4 < TB; t4 += 256) {
      const int dg = t4 % (HS / 4), kg = t4 / (HS / 4);
      uint2 a[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = j0 + kg * 4 + kk;
        a[kk] = key < T ? *reinterpret_cast<const uint2*>(Kg + head + (size_t)key * HS + dg * 4)
                        : make_uint2(0, 0);
      }
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const int sh = (dd & 1) * 16;
        uint2 o;
        o.x = (((dd < 2 ? a[0].x : a[0].y) >> sh) & 0xffffu) |
              ((((dd < 2 ? a[1].x : a[1].y) >> sh) & 0xffffu) << 16);
        o.y = (((dd < 2 ? a[2].x : a[2].y) >> sh) & 0xffffu) |
              ((((dd < 2 ? a[3].x : a[3].y) >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint2*>(&Kt[(dg * 4 + dd) * P2 + kg * 4]) = o;
      }
    }
    __syncthreads();

    if (j0 <= q0 + 31) {
      floatx16 s[2], dp[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kt][r] = 0.f;
          dp[kt][r] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < HS / 16; ++kk) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
              &Ks[(kt * 32 + (lane & 31)) * P1 + 16 * kk + 8 * hi]);
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(
              &Vs[(kt * 32 + (lane & 31)) * P1 + 16 * kk + 8 * hi]);
          s[kt] = mfma32(ka, qf[kk], s[kt]);
          dp[kt] = mfma32(va, gf[kk], dp[kt]);
        }
        uint4 wz[4];  // DROP: words of the 4 consecutive keys of each register group
        if constexpr (DROP) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            wz[g] = philox4x32_10(
                make_uint4((uint32_t)(j0 + kt * 32 + 8 * g + 4 * hi) >> 2, (uint32_t)myq,
                           (uint32_t)bh, 1u),
                drop.k0, drop.k1);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          float p = __builtin_amdgcn_exp2f(s[kt][r] * scale_log2 - L2);
          if (key > myq || myq >= T) p = 0.f;
          if constexpr (DROP) {
            const uint4 w = wz[r >> 2];
            const uint32_t wd = (r & 3) == 0 ? w.x : (r & 3) == 1 ? w.y : (r & 3) == 2 ? w.z : w.w;
            dp[kt][r] = p * (dp[kt][r] * (wd >= drop.thresh ? drop.scale : 0.f) - Dq);
          } else {
            dp[kt][r] = p * (dp[kt][r] - Dq);
          }
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8 sf;
#pragma unroll
          for (int e = 0; e < 8; ++e) sf[e] = (__bf16)dp[kt][8 * u + e];
          const int kb = kt * 32 + 16 * u + 4 * hi;
#pragma unroll
          for (int dt = 0; dt < HS / 32; ++dt) {
            const int drow = (dt * 32 + (lane & 31)) * P2 + kb;
            const uint2 lo = *reinterpret_cast<const uint2*>(&Kt[drow]);
            const uint2 up = *reinterpret_cast<const uint2*>(&Kt[drow + 8]);
            uint4 w;
            w.x = lo.x; w.y = lo.y; w.z = up.x; w.w = up.y;
            dq[dt] = mfma32(__builtin_bit_cast(bf16x8, w), sf, dq[dt]);
          }
        }
    }
    __syncthreads();
  }

  if (myq < T) {
    bf16_t* row = dqkv + ((size_t)b * T + myq) * 3 * C + (size_t)h * HS;
#pragma unroll
    for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        uint2 w;
        w.x = pack_bf16x2(dq[dt][4 * g] * scale, dq[dt][4 * g + 1] * scale);
        w.y = pack_bf16x2(dq[dt][4 * g + 2] * scale, dq[dt][4 * g + 3] * scale);
        *reinterpret_cast<uint2*>(row + d0) = w;
      }
  }
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
// out[i..i+3] = sum_k part[k][i..i+3] (n, stride multiples of 4; 16-byte
// partial loads).
__global__ __launch_bounds__(256) void reduce_partials4_bf16_kernel(
    const float* __restrict__ part, int S, size_t n, size_t stride, bf16_t* __restrict__ out) {
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n;
       i += (size_t)gridDim.x * 256 * 4) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < S; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(part + (size_t)k * stride + i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    uint2 w;
    w.x = pack_bf16x2(s.x, s.y);
    w.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<uint2*>(out + i) = w;
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

}  // namespace gpt_attn
