// skinny.cuh -- projection of at most 16 rows on the matrix cores (the
// decode step's projections and short-sequence forwards).
#pragma once

#include "common.cuh"

namespace gpt_attn {

constexpr int kDecCols = 16;     // output columns per skinny-GEMM block

// A block of a small-batch projection out[b][n] = sum_c x[b][c] W[c][n] for
// b < 16 and kDecCols = 16 columns n, on the matrix cores:
// v_mfma_f32_16x16x32_bf16 with A = the W slice transposed (16 columns n x 32
// rows c) and B = x transposed (32 rows c x 16 batch rows b), so that
// D[i][j] = out[j][n0 + i] and the sum over c runs inside the MFMA.  The rows
// go in k-steps of 32; wave w takes the steps w, w + 8, ..., kDecBatchSteps
// at a time, and copies the W rows of those steps (32 B per row: 16 columns)
// into its own LDS slots with global_load_lds_dwordx4 (one 1 KB load per
// step), so it needs no barrier before reading them: lane l of 16-lane group
// G = l / 16 reads, with ds_read_b64_tr_b16, rows 8G + 4t + (l % 16) / 4
// (t = 0, 1) at column 4 (l % 4) of the step, which hands it the A operand
// (column l % 16, rows 8G .. 8G + 7).  Its B operand, x[b][8G .. 8G + 7] with b = l % 16, is one
// 16-byte load.  The 8 waves' 16 x 16 accumulators are summed in LDS (fixed
// order: deterministic); the caller applies its epilogue.
constexpr int kDecWaves = 8;
constexpr int kDecBatchSteps = 4;   // k-steps whose x operands are loaded together

__device__ __align__(16) static const uint4 g_dec_zero16 = {0u, 0u, 0u, 0u};

// LDS bytes of one skinny-GEMM block: the waves' accumulators and W slots.
__host__ __device__ constexpr size_t skinny_lds_bytes() {
  return (size_t)kDecWaves * 64 * 4 * sizeof(float) + (size_t)kDecWaves * kDecBatchSteps * 1024;
}

// The MFMA part of a skinny-GEMM block: this wave's share of
// D[i][j] = sum_c W[c][n0 + i] x[j][c] (i, j < 16; rows j >= B read as 0),
// summed over the 8 waves into red[0][lane][r] (lane l, register r hold
// D[4 (l / 16) + r][l % 16]) before the block's barrier returns.
__device__ __forceinline__ void skinny_mfma(const bf16_t* __restrict__ x, int ldx, int B, int K,
                                            const bf16_t* __restrict__ W, int N, int n0,
                                            char* dsm) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  float* red = reinterpret_cast<float*>(dsm);                     // [kDecWaves][64][4]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // this wave's W slots: kDecBatchSteps k-steps of [32 rows][32 B]
  char* wslot = dsm + kDecWaves * 64 * 4 * sizeof(float) + w * kDecBatchSteps * 1024;
  const int nsteps = (K + 31) / 32;
  const int bj = lane & 15, g = lane >> 4;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int st0 = w; st0 < nsteps; st0 += kDecWaves * kDecBatchSteps) {
    // W rows of this batch's steps -> the wave's slots (lane -> row lane / 2,
    // 8 columns at 8 (lane % 2)), and the x operands
#pragma unroll
    for (int q = 0; q < kDecBatchSteps; ++q) {
      const int st = st0 + q * kDecWaves;
      if (st < nsteps) {
        const int row = st * 32 + (lane >> 1);
        const bf16_t* src = row < K ? W + (size_t)row * N + n0 + 8 * (lane & 1)
                                    : reinterpret_cast<const bf16_t*>(&g_dec_zero16);
        __builtin_amdgcn_load_to_lds(
            (void*)src, (__attribute__((address_space(3))) void*)(wslot + q * 1024), 16, 0, 0);
      }
    }
    bf16x8 xf[kDecBatchSteps];
#pragma unroll
    for (int q = 0; q < kDecBatchSteps; ++q) {
      const int st = st0 + q * kDecWaves, k = st * 32 + 8 * g;
      xf[q] = (st < nsteps && bj < B && k < K)
                  ? *reinterpret_cast<const bf16x8*>(x + (size_t)bj * ldx + k)
                  : bf16x8{};
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads have landed
#pragma unroll
    for (int q = 0; q < kDecBatchSteps; ++q) {
      const int st = st0 + q * kDecWaves;
      if (st >= nsteps) break;
      v4i16 r[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        r[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(wslot + q * 1024 +
                                                       (8 * g + 4 * t + (bj >> 2)) * 32 +
                                                       (bj & 3) * 8));
      const v8i16 av = {r[0][0], r[0][1], r[0][2], r[0][3], r[1][0], r[1][1], r[1][2], r[1][3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), xf[q], acc,
                                                    0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slots read before the next batch
  }
  *reinterpret_cast<floatx4*>(red + (w * 64 + lane) * 4) = acc;
  __syncthreads();
  // waves 1..7 into wave 0's slots, fixed order (lanes 0..63 x 4 registers)
  if (threadIdx.x < 256) {
    const int l = threadIdx.x >> 2, r = threadIdx.x & 3;
    float v = red[l * 4 + r];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) v += red[(ww * 64 + l) * 4 + r];
    red[l * 4 + r] = v;
  }
  __syncthreads();
}

}  // namespace gpt_attn
