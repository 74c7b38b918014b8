// gemm.cuh -- tiled GEMM kernels for gfx950 with fused epilogues.
//
// C[m][n] = sum_k A(m,k) * B(k,n), handed to an epilogue functor in chunks of
// 8 consecutive columns of one row.  Operand layouts are template choices:
//   A_KC = true : A(m,k) = A[m*lda + k]   (k contiguous, e.g. x [M][C])
//   A_KC = false: A(m,k) = A[k*lda + m]   (m contiguous, e.g. x^T in dW = x^T g)
//   B_KC = true : B(k,n) = B[n*ldb + k]   (k contiguous, e.g. W^T in dx = g W^T)
//   B_KC = false: B(k,n) = B[k*ldb + n]   (n contiguous, e.g. W [C][3C])
//
// bf16 path: 256 threads (4 waves as 2 x 2), block tile BM x BN, BK = 64,
// 32x32x16 bf16 MFMA with fp32 accumulators.  Both operands are staged in LDS
// k-contiguous ([row][k], padded pitch), so every MFMA operand is one 16-byte
// LDS read; m- or n-contiguous sources are transposed in registers on the
// way into LDS (4 k x 8 rows per thread).  Global loads for tile k+1 are
// issued before the MFMAs of tile k (two LDS buffers, one barrier per step).
// The accumulator tile is staged through LDS in fp32 so the epilogue sees
// whole rows and writes 16-byte vectors.
//
// fp32 path: plain LDS-tiled FMA kernel (64 x 64 tile, 4 x 4 per thread), used
// only for the fp32 element type.
#pragma once

#include "common.cuh"

namespace gpt_attn {

// ---------------------------------------------------------------- stores
__device__ __forceinline__ void store8(bf16_t* dst, const float* v) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(dst) = u;
}
__device__ __forceinline__ void store8(float* dst, const float* v) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
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
  __device__ __forceinline__ void operator()(int m, int n, const float* acc) const {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = acc[i] + (bias ? load1(bias + n + i) : 0.f);
    store8(out + (size_t)m * ldc + n, v);
  }
  __device__ __forceinline__ void one(int m, int n, float acc) const {
    store1(out + (size_t)m * ldc + n, acc + (bias ? load1(bias + n) : 0.f));
  }
};

// c_attn epilogue: adds the bias and scatters column n of row m = b*T + t to
// the head-major q/k/v buffer qkv[s][b][h][t][d] with s = n / C (0 q, 1 k,
// 2 v), h = (n % C) / hs, d = n % hs.  hs is a multiple of 8, so the 8
// columns of a chunk never straddle a head.
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
  __device__ __forceinline__ void operator()(int m, int n, const float* acc) const {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = acc[i] + (bias ? load1(bias + n + i) : 0.f);
    store8(dst(m, n), v);
  }
  __device__ __forceinline__ void one(int m, int n, float acc) const {
    store1(dst(m, n), acc + (bias ? load1(bias + n) : 0.f));
  }
};

// Split-K partial sums: split blockIdx.y writes its fp32 partial tile to
// part + blockIdx.y * split_stride (row-major, row stride ldc).
struct EpiPartial {
  float* part;
  int ldc;
  size_t split_stride;
  __device__ __forceinline__ void operator()(int m, int n, const float* acc) const {
    store8(part + (size_t)blockIdx.y * split_stride + (size_t)m * ldc + n, acc);
  }
  __device__ __forceinline__ void one(int m, int n, float acc) const {
    part[(size_t)blockIdx.y * split_stride + (size_t)m * ldc + n] = acc;
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

// ============================================================ bf16 MFMA
constexpr int kGemmBK = 64;
constexpr int kGemmLdk = kGemmBK + 8;  // LDS pitch (elements): 144 B rows

// Loads a ROWS x BK operand tile whose source is k-contiguous:
// element (row, k) at src[row*ld + k].  Rows >= nrows and k >= K read as 0.
// Requires K % 8 == 0.
template <int ROWS>
struct LoadKc {
  static constexpr int kChunks = ROWS * kGemmBK / 8;
  static constexpr int kPer = kChunks / 256;
  static_assert(kChunks % 256 == 0, "tile too small");
  uint4 r[kPer];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ src, int ld, int row0,
                                       int nrows, int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * 256;
      const int row = c / (kGemmBK / 8), kc = c % (kGemmBK / 8);
      const int gr = row0 + row, gk = k0 + kc * 8;
      if (gr < nrows && gk < K)
        r[i] = *reinterpret_cast<const uint4*>(src + (size_t)gr * ld + gk);
      else
        r[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * 256;
      const int row = c / (kGemmBK / 8), kc = c % (kGemmBK / 8);
      *reinterpret_cast<uint4*>(lds + row * kGemmLdk + kc * 8) = r[i];
    }
  }
};

// Loads a ROWS x BK operand tile whose source is row-contiguous:
// element (row, k) at src[k*ld + row], and writes it to LDS transposed
// ([row][k]).  Each thread owns 4 k x 8 rows.  Requires nrows % 8 == 0.
template <int ROWS>
struct LoadRc {
  static constexpr int kBlocks = (kGemmBK / 4) * (ROWS / 8);
  static constexpr int kPer = kBlocks / 256;
  static_assert(kBlocks % 256 == 0, "tile too small");
  uint4 r[kPer][4];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ src, int ld, int row0,
                                       int nrows, int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int blk = tid + i * 256;
      const int rg = blk % (ROWS / 8), kg = blk / (ROWS / 8);
      const int gr = row0 + rg * 8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int gk = k0 + kg * 4 + kk;
        if (gr < nrows && gk < K)
          r[i][kk] = *reinterpret_cast<const uint4*>(src + (size_t)gk * ld + gr);
        else
          r[i][kk] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  // 16-bit element e (0..7) of a 16-byte vector
  __device__ __forceinline__ static uint32_t half(const uint4& v, int e) {
    const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int blk = tid + i * 256;
      const int rg = blk % (ROWS / 8), kg = blk / (ROWS / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 o;
        o.x = half(r[i][0], e) | (half(r[i][1], e) << 16);
        o.y = half(r[i][2], e) | (half(r[i][3], e) << 16);
        *reinterpret_cast<uint2*>(lds + (rg * 8 + e) * kGemmLdk + kg * 4) = o;
      }
    }
  }
};

template <int ROWS, bool KC>
struct LoaderSel;
template <int ROWS>
struct LoaderSel<ROWS, true> { using type = LoadKc<ROWS>; };
template <int ROWS>
struct LoaderSel<ROWS, false> { using type = LoadRc<ROWS>; };

template <int BM, int BN>
struct GemmSmem {
  static constexpr int kOperand = 2 * (BM + BN) * kGemmLdk * 2;  // bytes, 2 buffers
  static constexpr int kStage = BM * (BN + 4) * 4;                // fp32 C tile
  static constexpr int kBytes = kOperand > kStage ? kOperand : kStage;
};

template <int BM, int BN, bool A_KC, bool B_KC, class Epi>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ Bm, int ldb,
    int M, int N, int K, int k_split, Epi epi) {
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must be a multiple of 64");
  constexpr int WTM = BM / 2, WTN = BN / 2;  // per-wave tile
  constexpr int MT = WTM / 32, NT = WTN / 32;
  __shared__ __align__(16) char smem[GemmSmem<BM, BN>::kBytes];
  bf16_t* As = reinterpret_cast<bf16_t*>(smem);
  bf16_t* Bs = As + 2 * BM * kGemmLdk;

  const int tiles_n = (N + BN - 1) / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  typename LoaderSel<BM, A_KC>::type la;
  typename LoaderSel<BN, B_KC>::type lb;
  // this block's slice of the reduction dimension: [kbeg, kend)
  const int kbeg = (int)blockIdx.y * k_split;
  const int kend = min(K, kbeg + k_split);
  const int nk = (kend - kbeg + kGemmBK - 1) / kGemmBK;

  floatx16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  la.load(A, lda, m0, M, kbeg, kend, tid);
  lb.load(Bm, ldb, n0, N, kbeg, kend, tid);
  la.store(As, tid);
  lb.store(Bs, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, lda, m0, M, kbeg + (kt + 1) * kGemmBK, kend, tid);
      lb.load(Bm, ldb, n0, N, kbeg + (kt + 1) * kGemmBK, kend, tid);
    }
    const bf16_t* as = As + buf * BM * kGemmLdk;
    const bf16_t* bs = Bs + buf * BN * kGemmLdk;
#pragma unroll
    for (int kk = 0; kk < kGemmBK / 16; ++kk) {
      bf16x8 af[MT], bfr[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(
            as + (wm * WTM + i * 32 + (lane & 31)) * kGemmLdk + kk * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(
            bs + (wn * WTN + j * 32 + (lane & 31)) * kGemmLdk + kk * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      la.store(As + (buf ^ 1) * BM * kGemmLdk, tid);
      lb.store(Bs + (buf ^ 1) * BN * kGemmLdk, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: stage the fp32 tile in LDS, then hand out 8-column chunks
  float* Cs = reinterpret_cast<float*>(smem);
  constexpr int CP = BN + 4;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * WTN + j * 32 + (lane & 31);
        Cs[row * CP + col] = acc[i][j][r];
      }
  __syncthreads();
  constexpr int kChunks = BM * BN / 8;
#pragma unroll
  for (int c = tid; c < kChunks; c += 256) {
    const int row = c / (BN / 8), cc = c % (BN / 8);
    const int gm = m0 + row, gn = n0 + cc * 8;
    if (gm < M && gn < N) {
      float v[8];
      const float4 a = *reinterpret_cast<const float4*>(Cs + row * CP + cc * 8);
      const float4 b = *reinterpret_cast<const float4*>(Cs + row * CP + cc * 8 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      epi(gm, gn, v);
    }
  }
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
// splits > 1 divides K into that many slices of a multiple of 64 (the
// epilogue then must be EpiPartial); returns the number of slices launched.
template <int BM, int BN, bool A_KC, bool B_KC, class Epi>
inline int launch_gemm_bf16(const bf16_t* A, int lda, const bf16_t* B, int ldb, int M,
                            int N, int K, const Epi& epi, hipStream_t st, int splits = 1) {
  const int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (grid == 0 || K <= 0) return 0;
  if (splits < 1) splits = 1;
  int k_split = (K + splits - 1) / splits;
  k_split = (k_split + kGemmBK - 1) / kGemmBK * kGemmBK;
  const int ns = (K + k_split - 1) / k_split;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, A_KC, B_KC, Epi>), dim3(grid, ns), dim3(256), 0,
                     st, A, lda, B, ldb, M, N, K, k_split, epi);
  return ns;
}

template <bool A_KC, bool B_KC, class Epi>
inline void launch_gemm_f32(const float* A, int lda, const float* B, int ldb, int M, int N,
                            int K, const Epi& epi, hipStream_t st) {
  const int grid = ((M + 63) / 64) * ((N + 63) / 64);
  if (grid == 0) return;
  hipLaunchKernelGGL((gemm_f32_kernel<A_KC, B_KC, Epi>), dim3(grid), dim3(256), 0, st, A,
                     lda, B, ldb, M, N, K, epi);
}

}  // namespace gpt_attn
