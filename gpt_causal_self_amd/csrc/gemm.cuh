// gemm.cuh -- the fp32 GEMM of the fp32 element type, the epilogues it
// shares with the fp32 attention path, and the XCD-aware block -> tile map.
//
// C[m][n] = sum_k A(m,k) * B(k,n), handed to an epilogue functor element by
// element.  Operand layouts are template choices:
//   A_KC = true : A(m,k) = A[m*lda + k]   (k contiguous, e.g. x [M][C])
//   A_KC = false: A(m,k) = A[k*lda + m]   (m contiguous, e.g. x^T in dW = x^T g)
//   B_KC = true : B(k,n) = B[n*ldb + k]   (k contiguous, e.g. W^T in dx = g W^T)
//   B_KC = false: B(k,n) = B[k*ldb + n]   (n contiguous, e.g. W [C][3C])
// Plain LDS-tiled FMA kernel (64 x 64 tile, 4 x 4 per thread).  The bf16
// matrix-core GEMM is gemm2.cuh.
#pragma once

#include "common.cuh"

namespace gpt_attn {

// ---------------------------------------------------------------- stores
__device__ __forceinline__ void store1(bf16_t* dst, float v) { *dst = f2bf(v); }
__device__ __forceinline__ void store1(float* dst, float v) { *dst = v; }
__device__ __forceinline__ float load1(const bf16_t* p) { return bf2f(*p); }
__device__ __forceinline__ float load1(const float* p) { return *p; }

// ------------------------------------------------------------- epilogues
// Row-major output with optional bias: out[m*ldc + n] = acc + bias[n].
template <class OutT>
struct EpiRowMajor {
  OutT* out;
  int ldc;
  const OutT* bias;  // may be NULL
  __device__ __forceinline__ void one(int m, int n, float acc) const {
    store1(out + (size_t)m * ldc + n, acc + (bias ? load1(bias + n) : 0.f));
  }
};

// c_attn epilogue: adds the bias and scatters column n of row m = b*T + t to
// the head-major q/k/v buffer qkv[s][b][h][t][d] with s = n / C (0 q, 1 k,
// 2 v), h = (n % C) / hs, d = n % hs.
template <class OutT>
struct EpiQKV {
  OutT* qkv;
  const OutT* bias;  // [3C] or NULL
  int B, T, C, H, hs;
  __device__ __forceinline__ OutT* dst(int m, int n) const {
    const int s = n / C, rem = n - s * C;
    const int h = rem / hs, d = rem - h * hs;
    const int b = m / T, t = m - b * T;
    return qkv + ((((size_t)s * B + b) * H + h) * T + t) * hs + d;
  }
  __device__ __forceinline__ void one(int m, int n, float acc) const {
    store1(dst(m, n), acc + (bias ? load1(bias + n) : 0.f));
  }
};

// Block index -> tile index so that the blocks a given XCD receives (the
// dispatcher deals block ids round-robin over the 8 XCDs) form one
// contiguous run of tiles; neighbouring tiles then share an L2.
__device__ __forceinline__ int xcd_swizzle(int bid, int nb) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd, idx = bid / kXcd;
  const int per = nb / kXcd, extra = nb % kXcd;
  return xcd < extra ? xcd * (per + 1) + idx
                     : extra * (per + 1) + (xcd - extra) * per + idx;
}

// ============================================================ fp32 FMA
// 64 x 64 tile, 16 x 16 threads with 4 x 4 outputs each, BK = 32.  The next
// k-tile's global loads are issued into registers before the current tile's
// FMAs and land in the other half of a double-buffered LDS tile, so each
// step waits for its loads only after a tile of arithmetic and needs one
// barrier.  Consecutive threads load consecutive addresses: along k for a
// k-contiguous operand, along the rows otherwise.
template <bool A_KC, bool B_KC, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int lda, const float* __restrict__ Bm, int ldb, int M,
    int N, int K, Epi epi) {
  constexpr int BM = 64, BN = 64, BK = 32;
  constexpr int PER = BK * BM / 256;  // elements of each operand per thread per k-tile
  __shared__ float As[2][BK][BM + 4];
  __shared__ float Bs[2][BK][BN + 4];
  const int tiles_n = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
  const int tid = threadIdx.x;
  const int tm = tid / 16, tn = tid % 16;
  float acc[4][4] = {};
  float ra[PER], rb[PER];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + 256 * i;
      const int ka = A_KC ? e % BK : e / BM, ma = A_KC ? e / BK : e % BM;
      const int kb = B_KC ? e % BK : e / BN, nb = B_KC ? e / BK : e % BN;
      const int gm = m0 + ma, gka = k0 + ka, gn = n0 + nb, gkb = k0 + kb;
      ra[i] = (gm < M && gka < K) ? (A_KC ? A[(size_t)gm * lda + gka] : A[(size_t)gka * lda + gm])
                                  : 0.f;
      rb[i] = (gn < N && gkb < K) ? (B_KC ? Bm[(size_t)gn * ldb + gkb] : Bm[(size_t)gkb * ldb + gn])
                                  : 0.f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + 256 * i;
      if (A_KC) As[buf][e % BK][e / BK] = ra[i];
      else As[buf][e / BM][e % BM] = ra[i];
      if (B_KC) Bs[buf][e % BK][e / BK] = rb[i];
      else Bs[buf][e / BN][e % BN] = rb[i];
    }
  };
  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool next = k0 + BK < K;
    if (next) load(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[buf][kk][tm * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[buf][kk][tn * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    if (next) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gm = m0 + tm * 4 + i, gn = n0 + tn * 4 + j;
      if (gm < M && gn < N) epi.one(gm, gn, acc[i][j]);
    }
}

// ------------------------------------------------------------- launchers
template <bool A_KC, bool B_KC, class Epi>
inline void launch_gemm_f32(const float* A, int lda, const float* B, int ldb, int M, int N,
                            int K, const Epi& epi, hipStream_t st) {
  const int grid = ((M + 63) / 64) * ((N + 63) / 64);
  if (grid == 0) return;
  hipLaunchKernelGGL((gemm_f32_kernel<A_KC, B_KC, Epi>), dim3(grid), dim3(256), 0, st, A,
                     lda, B, ldb, M, N, K, epi);
}

}  // namespace gpt_attn
