// decode.cuh -- one-token decode of the causal self-attention layer against a
// key/value cache.
//
// The pages' generate() re-runs the (cropped) prefix through the model for
// every new token and keeps only the last position (page "nanoGPT global
// flow walkthrough", fifth stage, GPT.generate); page "GPT architecture:
// design ideas and core concepts" names a KV cache as the inference
// optimisation.  Because the layer is causal, the last row of a full forward
// over positions 0..pos equals one token's step that reads the keys and
// values of positions 0..pos-1 from a cache: this file computes that step.
//
//   skinny_gemm_kernel   out[b][n] = sum_c x[b][c] W[c][n] (+ bias) for a
//                        handful of rows b (the batch); HBM-bound on W.  The
//                        epilogue either scatters q / k / v (q to a buffer,
//                        k and v into the caches at `pos`) or writes a
//                        row-major output.
//   decode_attn_kernel   per (b, h) and chunk of kChunk cached keys: scores,
//                        chunk max, exp2 weights, chunk sum and the weighted
//                        value sum (fp32 partials); HBM-bound on the cache.
//   decode_combine_kernel  merges the chunk partials (rescaling by the chunk
//                        maxima) and writes the merged heads in bf16.
#pragma once

#include "common.cuh"

namespace gpt_attn {

constexpr int kDecChunk = 256;   // cached keys per attention block
constexpr int kDecMaxB = 16;     // rows of one decode call
constexpr int kDecCols = 64;     // output columns per skinny-GEMM block

// q/k/v epilogue of the decode projection: column n of row b goes to
// q[b][n] (n < C), k_cache[b][h][pos][d] (C <= n < 2C) or v_cache (2C <= n).
struct DecQKVOut {
  bf16_t* q;         // [B][C]
  bf16_t* k_cache;   // [B][H][cache_T][hs]
  bf16_t* v_cache;
  int C, H, hs, cache_T, pos;
  __device__ __forceinline__ void put(int b, int n, float v) const {
    const bf16_t r = f2bf(v);
    if (n < C) { q[(size_t)b * C + n] = r; return; }
    const int s = n >= 2 * C ? 2 : 1;
    const int rem = n - s * C, h = rem / hs, d = rem - h * hs;
    bf16_t* cache = s == 1 ? k_cache : v_cache;
    cache[(((size_t)b * H + h) * cache_T + pos) * hs + d] = r;
  }
};

struct DecRowOut {
  bf16_t* y;  // [B][N]
  int N;
  __device__ __forceinline__ void put(int b, int n, float v) const {
    y[(size_t)b * N + n] = f2bf(v);
  }
};

// partial[y][b][n] = sum_{c in slice y} x[b][c] W[c][n] for b < B (<=
// kDecMaxB), n in this block's kDecCols columns, the K rows split into
// gridDim.y slices (skinny_finish_kernel adds the slices, the bias and
// applies the epilogue).  512 threads = 8 waves; in a wave
// lane = ks + 8 * cg: cg picks 8 consecutive columns (16-byte loads; the 8
// lanes of one ks read one 128-byte row run) and the row slot r = 8 * w + ks
// takes the rows c = r, r + 64, ...; loads are issued kDecUnroll rows at a
// time so that several are in flight per lane.  Partial sums are reduced
// across the 8 row slots of a wave with DPP lane moves and across the 8 waves
// in LDS (fixed order: the result is deterministic).  x is staged in LDS as
// bf16.
constexpr int kDecWaves = 8;
constexpr int kDecUnroll = 8;
constexpr int kDecKSplit = 4;   // row slices of a decode projection

__global__ __launch_bounds__(64 * kDecWaves) void skinny_gemm_kernel(
    const bf16_t* __restrict__ x, int B, int K, const bf16_t* __restrict__ W, int N,
    float* __restrict__ partial) {
  extern __shared__ float dsm[];
  float* red = dsm;                                                   // [8][B][kDecCols]
  bf16_t* xs = reinterpret_cast<bf16_t*>(dsm + kDecWaves * B * kDecCols);  // [B][K], 16-B aligned
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < B * K / 8; i += 64 * kDecWaves)  // K % 8 == 0: 16-byte chunks
    reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(x)[i];
  __syncthreads();
  const int ks = lane & 7, cg = lane >> 3;
  const int n = blockIdx.x * kDecCols + 8 * cg;
  constexpr int kSlots = 8 * kDecWaves;
  float acc[kDecMaxB][8];
#pragma unroll
  for (int b = 0; b < kDecMaxB; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
  // this block's slice of the rows: [kb, ke)
  const int KS = gridDim.y;
  const int kb = (int)(((long)K * blockIdx.y) / KS), ke = (int)(((long)K * (blockIdx.y + 1)) / KS);
  if (n < N) {
    for (int c0 = kb + 8 * w + ks; c0 < ke; c0 += kSlots * kDecUnroll) {
      uint4 u[kDecUnroll];
#pragma unroll
      for (int q = 0; q < kDecUnroll; ++q) {
        const int c = c0 + q * kSlots;
        u[q] = c < ke ? *reinterpret_cast<const uint4*>(W + (size_t)c * N + n)
                      : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int q = 0; q < kDecUnroll; ++q) {
        const int c = c0 + q * kSlots;
        if (c >= ke) break;
        const unsigned wd[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
        float wf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wf[2 * e] = bf2f(wd[e] & 0xffff);
          wf[2 * e + 1] = bf2f(wd[e] >> 16);
        }
#pragma unroll
        for (int b = 0; b < kDecMaxB; ++b) {
          if (b < B) {
            const float xv = bf2f(xs[b * K + c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[b][e] = fmaf(xv, wf[e], acc[b][e]);
          }
        }
      }
    }
  }
  // sum over the 8 row slots of a column group (8 consecutive lanes) with
  // DPP moves: swap neighbours, swap pairs (every lane of a quad then holds
  // the quad's sum), then add the mirrored lane of the half-row (the other
  // quad): every lane of the group ends with the group's total
#pragma unroll
  for (int b = 0; b < kDecMaxB; ++b) {
    if (b < B) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[b][e];
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
        acc[b][e] = v;
      }
    }
  }
  if (ks == 0) {
#pragma unroll
    for (int b = 0; b < kDecMaxB; ++b)  // unrolled: acc stays in registers
      if (b < B)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[((size_t)w * B + b) * kDecCols + 8 * cg + e] = acc[b][e];
  }
  __syncthreads();
  // this slice's totals -> partial[slice][b][n]
  for (int i = tid; i < B * kDecCols; i += 64 * kDecWaves) {
    const int b = i / kDecCols, col = i - b * kDecCols;
    const int nn = blockIdx.x * kDecCols + col;
    if (nn >= N) continue;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) v += red[(ww * B + b) * kDecCols + col];
    partial[((size_t)blockIdx.y * B + b) * N + nn] = v;
  }
}

// out.put(b, n, sum_y partial[y][b][n] + bias[n]): the fixed-order sum of the
// row slices of skinny_gemm_kernel (deterministic), one thread per output.
template <class Out>
__global__ __launch_bounds__(256) void skinny_finish_kernel(const float* __restrict__ partial,
                                                            int KS, int B, int N,
                                                            const bf16_t* __restrict__ bias,
                                                            Out out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B * N) return;
  const int b = i / N, n = i - b * N;
  float v = 0.f;
  for (int y = 0; y < KS; ++y) v += partial[((size_t)y * B + b) * N + n];
  if (bias) v += bf2f(bias[n]);
  out.put(b, n, v);
}

// Attention of one query per (b, h) over cached keys [chunk * kDecChunk,
// min(pos + 1, (chunk + 1) * kDecChunk)).  One thread per key for the scores;
// the weighted value sum gives each thread 8 value columns of a few keys.  Writes (m, l, o[0..HS)) in fp32, with
// m the chunk's max of the log2-scaled scores, l = sum 2^(s - m) and
// o = sum 2^(s - m) v.
template <int HS>
__global__ __launch_bounds__(256) void decode_attn_kernel(const bf16_t* __restrict__ q,
                                                          const bf16_t* __restrict__ k_cache,
                                                          const bf16_t* __restrict__ v_cache,
                                                          float* __restrict__ part, int H,
                                                          int cache_T, int pos, int nchunk,
                                                          float scale_log2) {
  __shared__ float ps[kDecChunk];
  __shared__ float wred[8];
  __shared__ float ored[256 / (HS / 8)][HS];
  const int bh = blockIdx.x, chunk = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int C = H * HS;
  float qf[HS];
#pragma unroll
  for (int d8 = 0; d8 < HS / 8; ++d8) {
    const uint4 u = *reinterpret_cast<const uint4*>(q + (size_t)b * C + h * HS + 8 * d8);
    const unsigned wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[8 * d8 + 2 * e] = bf2f(wd[e] & 0xffff);
      qf[8 * d8 + 2 * e + 1] = bf2f(wd[e] >> 16);
    }
  }
  const size_t head = ((size_t)b * H + h) * cache_T * HS;
  const int j = chunk * kDecChunk + tid;
  float s = -INFINITY;
  if (j <= pos) {
    const bf16_t* kr = k_cache + head + (size_t)j * HS;
    float acc = 0.f;
#pragma unroll
    for (int d8 = 0; d8 < HS / 8; ++d8) {
      const uint4 u = *reinterpret_cast<const uint4*>(kr + 8 * d8);
      const unsigned wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(qf[8 * d8 + 2 * e], bf2f(wd[e] & 0xffff), acc);
        acc = fmaf(qf[8 * d8 + 2 * e + 1], bf2f(wd[e] >> 16), acc);
      }
    }
    s = acc * scale_log2;
  }
  float m = s;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) wred[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  const float p = j <= pos ? __builtin_amdgcn_exp2f(s - m) : 0.f;
  ps[tid] = p;
  float l = p;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  if (lane == 0) wred[4 + w] = l;
  __syncthreads();
  l = wred[4] + wred[5] + wred[6] + wred[7];
  // weighted value sum: thread -> (key group kg, 8 value columns dg); each
  // thread reads its group's value rows with 16-byte loads, all in flight
  constexpr int DG = HS / 8, KG = 256 / DG, KPG = kDecChunk / KG;
  const int dg = tid % DG, kg = tid / DG;
  const int jb = chunk * kDecChunk + kg * KPG;
  uint4 vr[KPG];
#pragma unroll
  for (int u = 0; u < KPG; ++u)
    vr[u] = jb + u <= pos
                ? *reinterpret_cast<const uint4*>(v_cache + head + (size_t)(jb + u) * HS + 8 * dg)
                : make_uint4(0u, 0u, 0u, 0u);
  float o8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    const float pj = ps[kg * KPG + u];  // 0 beyond pos
    const unsigned wd[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o8[2 * e] = fmaf(pj, bf2f(wd[e] & 0xffff), o8[2 * e]);
      o8[2 * e + 1] = fmaf(pj, bf2f(wd[e] >> 16), o8[2 * e + 1]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) ored[kg][8 * dg + e] = o8[e];
  __syncthreads();
  if (tid < HS) {
    float t = 0.f;
    for (int g = 0; g < KG; ++g) t += ored[g][tid];
    float* pr = part + ((size_t)bh * nchunk + chunk) * (HS + 2);
    pr[2 + tid] = t;
    if (tid == 0) {
      pr[0] = m;
      pr[1] = l;
    }
  }
}

// Merge the chunk partials of each (b, h): y_m[b][h*HS + d] = bf16(o / l)
// with every chunk rescaled to the common maximum.
template <int HS>
__global__ __launch_bounds__(HS) void decode_combine_kernel(const float* __restrict__ part,
                                                            bf16_t* __restrict__ ym, int H,
                                                            int nchunk) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const int b = bh / H, h = bh - b * H;
  const float* pr = part + (size_t)bh * nchunk * (HS + 2);
  float m = -INFINITY;
  for (int c = 0; c < nchunk; ++c) m = fmaxf(m, pr[c * (HS + 2)]);
  float l = 0.f, o = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const float a = __builtin_amdgcn_exp2f(pr[c * (HS + 2)] - m);
    l = fmaf(pr[c * (HS + 2) + 1], a, l);
    o = fmaf(pr[c * (HS + 2) + 2 + d], a, o);
  }
  ym[(size_t)b * H * HS + h * HS + d] = f2bf(o / l);
}

// Copy the keys and values of positions [0, T) from the head-major q/k/v
// workspace of a forward ([3][B][H][T][hs]) into caches [B][H][cache_T][hs].
__global__ void export_kv_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                 bf16_t* __restrict__ k_cache, bf16_t* __restrict__ v_cache,
                                 int BH, int T, int hs, int cache_T) {
  const size_t per = (size_t)T * hs / 8;  // 16-byte chunks per (b, h)
  const size_t total = (size_t)BH * per;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = i / per, r = i - bh * per;
    const size_t src = bh * T * hs + r * 8, dst = bh * (size_t)cache_T * hs + r * 8;
    *reinterpret_cast<uint4*>(k_cache + dst) = *reinterpret_cast<const uint4*>(k + src);
    *reinterpret_cast<uint4*>(v_cache + dst) = *reinterpret_cast<const uint4*>(v + src);
  }
}

// LDS bytes of one skinny-GEMM block.
inline size_t skinny_lds_bytes(int B, int K) {
  return (size_t)kDecWaves * B * kDecCols * sizeof(float) + (size_t)B * K * sizeof(bf16_t);
}

}  // namespace gpt_attn
