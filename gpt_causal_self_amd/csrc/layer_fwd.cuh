// layer_fwd.cuh -- launch sequence of the bf16 layer forward, shared by
// gpt_attn_forward and the Pre-LN block entry point.
#pragma once

#include <type_traits>

#include <algorithm>

#include "attn_fwd.cuh"
#include "gemm2.cuh"
#include "gemm3.cuh"
#include "skinny.cuh"
#include "handle.cuh"

namespace gpt_attn {

// bf16 residual run of 8 columns as fp32 helpers
__device__ __forceinline__ void bf16x8_to_f32(uint4 u, float* f) {
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf2f(w[e] & 0xffff);
    f[2 * e + 1] = bf2f(w[e] >> 16);
  }
}

// c_proj epilogue with the Block's residual (page "nanoGPT global flow
// walkthrough", section 2.5: the attention output is added back onto x):
// out = bf16(acc + bias + res), one rounding.  Through the GEMM's fp32
// staged epilogue (coalesced 16-byte runs; the residual runs of all passes
// are loaded before the stores) or called per 4 columns (split-K finish,
// short-sequence path).
struct Epi2RowMajorRes {
  bf16_t* out;
  int ldc;
  const bf16_t* bias;  // may be NULL
  const bf16_t* res;   // [M][ldc]
  static constexpr bool kStaged = true;
  static constexpr bool kStagedF32 = true;
  __device__ __forceinline__ const bf16_t* bias_ptr() const { return bias; }
  typedef uint4 Extra8;
  __device__ __forceinline__ Extra8 extra8(int m, int n, bool ok) const {
    return ok ? *reinterpret_cast<const uint4*>(res + (size_t)m * ldc + n)
              : make_uint4(0u, 0u, 0u, 0u);
  }
  // v: acc + bias of columns n .. n+7
  __device__ __forceinline__ void store8f(int m, int n, const float* v, const Extra8& r) const {
    float x[8];
    bf16x8_to_f32(r, x);
    uint4 o;
    o.x = pack_bf16x2(v[0] + x[0], v[1] + x[1]);
    o.y = pack_bf16x2(v[2] + x[2], v[3] + x[3]);
    o.z = pack_bf16x2(v[4] + x[4], v[5] + x[5]);
    o.w = pack_bf16x2(v[6] + x[6], v[7] + x[7]);
    store16_stream(out + (size_t)m * ldc + n, o);
  }
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
// optional residual: out = res + keep * (acc + bias) / (1 - p), one rounding;
// staged in fp32 like Epi2RowMajorRes, or called per 4 columns.  One Philox
// call per 4 columns.
struct Epi2RowMajorDrop {
  bf16_t* out;
  int ldc;
  const bf16_t* bias;  // may be NULL
  const bf16_t* res;   // may be NULL
  DropParams drop;
  static constexpr bool kStaged = true;
  static constexpr bool kStagedF32 = true;
  __device__ __forceinline__ const bf16_t* bias_ptr() const { return bias; }
  typedef uint4 Extra8;
  __device__ __forceinline__ Extra8 extra8(int m, int n, bool ok) const {
    return (ok && res) ? *reinterpret_cast<const uint4*>(res + (size_t)m * ldc + n)
                       : make_uint4(0u, 0u, 0u, 0u);
  }
  // out[m][n .. n+3] = r + keep * a * scale for 4 values a (bias included)
  __device__ __forceinline__ uint2 apply4(int m, int n, const float* a, const float* r) const {
    // columns n..n+3 (n % 4 == 0): one Philox call
    const uint4 w = philox4x32_10(make_uint4((uint32_t)n >> 2, (uint32_t)m, 0u, 2u), drop.k0,
                                  drop.k1);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = r[e] + (wd[e] >= drop.thresh ? a[e] * drop.scale : 0.f);
    uint2 st;
    st.x = pack_bf16x2(o[0], o[1]);
    st.y = pack_bf16x2(o[2], o[3]);
    return st;
  }
  // v: acc + bias of columns n .. n+7
  __device__ __forceinline__ void store8f(int m, int n, const float* v, const Extra8& rr) const {
    float x[8];
    bf16x8_to_f32(rr, x);
    const uint2 lo = apply4(m, n, v, x), hi = apply4(m, n + 4, v + 4, x + 4);
    store16_stream(out + (size_t)m * ldc + n, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    float a[4] = {v[0], v[1], v[2], v[3]};
    if (bias) {
      const uint2 u = *reinterpret_cast<const uint2*>(bias + n);
      a[0] += bf2f(u.x & 0xffff); a[1] += bf2f(u.x >> 16);
      a[2] += bf2f(u.y & 0xffff); a[3] += bf2f(u.y >> 16);
    }
    float r[4] = {0.f, 0.f, 0.f, 0.f};
    if (res) {
      const uint2 u = *reinterpret_cast<const uint2*>(res + (size_t)m * ldc + n);
      r[0] = bf2f(u.x & 0xffff); r[1] = bf2f(u.x >> 16);
      r[2] = bf2f(u.y & 0xffff); r[3] = bf2f(u.y >> 16);
    }
    *reinterpret_cast<uint2*>(out + (size_t)m * ldc + n) = apply4(m, n, a, r);
  }
};

// Split-K for a projection whose output tiles cannot fill the chip (short
// sequences: at B = 4, C = 1600 the c_attn GEMM has 19 tiles per 256 rows).
// The k-slices write fp32 partials [s][M][N] into the handle's partial
// buffer; splitk_finish_kernel sums them in slice order and hands the sums
// to the projection's own epilogue (bias, q/k/v scatter, residual, dropout),
// so the result differs from the single-pass GEMM only in the fp32 order of
// the k summation.
template <class Epi>
__global__ __launch_bounds__(256) void splitk_finish_kernel(const float* __restrict__ part,
                                                            int S, int M, int N, Epi epi) {
  const int n4 = N / 4;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)M * n4) return;
  const int m = (int)(i / n4), n = (int)(i - (long)m * n4) * 4;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(part + ((size_t)s * M + m) * N + n);
    v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w;
  }
  if constexpr (SplitOffsets<Epi>::value)
    epi.store(epi.row_off(m) + epi.col_off(n), n, v);
  else
    epi(m, n, v);
}

// A projection of at most a few dozen rows (a short sequence) on the matrix
// cores: the decode path's skinny block (16 columns over all K per block,
// the sum over K inside v_mfma_f32_16x16x32_bf16) over 16-row chunks
// (gridDim.y), each thread handing 4 consecutive columns of one row to the
// projection's own epilogue (bias, q/k/v scatter, residual, dropout).  A is
// k-contiguous [M][lda], B row-contiguous [K][ldb = N].
#ifndef GA_SKINNY_MAX_M
#define GA_SKINNY_MAX_M 16
#endif
template <class Epi>
__global__ __launch_bounds__(64 * kDecWaves) void skinny_epi_kernel(const bf16_t* __restrict__ A,
                                                                    int lda, int M, int K,
                                                                    const bf16_t* __restrict__ Bm,
                                                                    int N, Epi epi) {
  extern __shared__ __align__(16) char dsm[];
  const int n0 = blockIdx.x * kDecCols, m0 = blockIdx.y * 16;
  skinny_mfma(A + (size_t)m0 * lda, lda, min(16, M - m0), K, Bm, N, n0, dsm);
  const float* red = reinterpret_cast<const float*>(dsm);
  const int o = threadIdx.x;  // row j = o % 16, columns n0 + 4 (o / 16) + 0..3
  if (o < 64) {
    const int j = o & 15, q = o >> 4;
    const int m = m0 + j, n = n0 + 4 * q;
    if (m < M && n < N) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = red[(q * 16 + j) * 4 + r];
      if constexpr (SplitOffsets<Epi>::value)
        epi.store(epi.row_off(m) + epi.col_off(n), n, v);
      else
        epi(m, n, v);
    }
  }
}

// Whether a projection onto N columns over M rows takes gemm3's 96 x 384
// tiles: N a multiple of 384 (no partly empty column tile) and at least 128
// tiles (enough blocks without a split of K).
inline bool use_gemm3(int M, int N) {
  return N % 384 == 0 && (long)((M + 95) / 96) * (N / 384) >= 128;
}

// The projection GEMM, split along K when it has fewer than 128 output
// tiles: up to 8 slices (each at least 2 k-tiles), as many as give about
// 256 blocks and fit the partial buffer.
template <int BM, int BN, int NSTAGE, int BK, int WGM, int WGN, bool A_KC, bool B_KC,
          int OCC = 1, class Epi>
inline void launch_proj(const gpt_attn_handle* h, const bf16_t* A, int lda, const bf16_t* Bm,
                        int ldb, int M, int N, int K, const Epi& epi, hipStream_t st) {
  if constexpr (A_KC && !B_KC) {
    if (M <= GA_SKINNY_MAX_M && N % kDecCols == 0 && K % 8 == 0 && ldb == N) {
      hipLaunchKernelGGL(skinny_epi_kernel<Epi>, dim3(N / kDecCols, (M + 15) / 16),
                         dim3(64 * kDecWaves), skinny_lds_bytes(), st, A, lda, M, K, Bm, N, epi);
      return;
    }
  }
  if constexpr ((std::is_same<Epi, Epi2RowMajor>::value ||
                 std::is_same<Epi, Epi2RowMajorRes>::value ||
                 std::is_same<Epi, Epi2RowMajorDrop>::value) &&
                A_KC && !B_KC) {
    if (use_gemm3(M, N)) {
      launch_gemm3<GA_PROJ3_TILE, true, false>(A, lda, Bm, ldb, M, N, K, epi, st);
      return;
    }
  }
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int nk = (K + BK - 1) / BK;
  int s = tiles >= 128 ? 1 : std::min(std::min(256 / std::max(tiles, 1), nk / 2), 8);
  while (s > 1 && (size_t)s * M * N > h->part_elems) --s;
  if (s <= 1) {
    launch_gemm2<BM, BN, NSTAGE, BK, WGM, WGN, A_KC, B_KC, OCC>(A, lda, Bm, ldb, M, N, K, epi,
                                                                st);
    return;
  }
  Epi2Partial ep{h->part, N, (size_t)M * N};
  const int ns = launch_gemm2<BM, BN, NSTAGE, BK, WGM, WGN, A_KC, B_KC, OCC>(
      A, lda, Bm, ldb, M, N, K, ep, st, s);
  const long total = (long)M * (N / 4);
  hipLaunchKernelGGL(splitk_finish_kernel<Epi>, dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, st, (const float*)h->part, ns, M, N, epi);
}

// c_attn GEMM -> fused causal attention -> c_proj GEMM on stream st.
// residual == NULL: y = layer(x); else y = residual + layer(x).
// lse != NULL: also store the softmax log-sum-exp rows for the backward.
// drop != NULL: dropout on the attention weights and the c_proj output;
// keepq / keepk != NULL: also store the attention weights' keep bits
// (keep_bits.cuh) for the backward.
inline void layer_forward_bf16(const gpt_attn_handle* h, const bf16_t* x, int B, int T,
                               const bf16_t* W_attn, const bf16_t* b_attn,
                               const bf16_t* W_proj, const bf16_t* b_proj, bf16_t* y,
                               const bf16_t* residual, float* lse, hipStream_t st,
                               const DropParams* drop = nullptr, uint32_t* keepq = nullptr,
                               uint16_t* keepk = nullptr) {
  const int C = h->C, H = h->H, hs = h->hs;
  const int M = B * T;
  const size_t head_elems = (size_t)B * H * T * hs;  // one of q, k, v
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)hs));
  bf16_t* qkv = (bf16_t*)h->qkv;
  bf16_t* o = (bf16_t*)h->o;
  Epi2QKV e1{qkv, b_attn, B, T, C, H, hs, 3 * head_elems * 2 < (size_t)1 << 31};
  mark(h, 0, st);
  launch_proj<GA_QKV_TILE, true, false, GA_QKV_OCC>(h, x, C, W_attn, 3 * C, M, 3 * C, C, e1, st);
  mark(h, 1, st);
  const dim3 agrid(B * H, (T + kAttnBQ - 1) / kAttnBQ);
  if (drop) {
    if (hs == 64)
      hipLaunchKernelGGL((attn_fwd2_bf16_kernel<64, GA_ATTN_STAGES, true>), agrid, dim3(256), 0,
                         st, qkv, qkv + head_elems, qkv + 2 * head_elems, o, lse, H, T,
                         scale_log2, *drop, keepq, keepk);
    else
      hipLaunchKernelGGL((attn_fwd2_bf16_kernel<32, GA_ATTN_STAGES, true>), agrid, dim3(256), 0,
                         st, qkv, qkv + head_elems, qkv + 2 * head_elems, o, lse, H, T,
                         scale_log2, *drop, keepq, keepk);
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
    launch_proj<GA_PROJ_TILE, true, false>(h, o, C, W_proj, C, M, C, C, e3, st);
  } else if (residual) {
    Epi2RowMajorRes e3{y, C, b_proj, residual};
    launch_proj<GA_PROJ_TILE, true, false>(h, o, C, W_proj, C, M, C, C, e3, st);
  } else {
    Epi2RowMajor e3{y, C, b_proj};
    launch_proj<GA_PROJ_TILE, true, false>(h, o, C, W_proj, C, M, C, C, e3, st);
  }
  mark(h, 3, st);
}

}  // namespace gpt_attn
