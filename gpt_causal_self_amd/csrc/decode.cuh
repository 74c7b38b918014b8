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
//                        handful of rows b (the batch, <= 16); HBM-bound on
//                        W.  A block takes 16 columns over all rows c on the
//                        matrix cores and applies the epilogue itself, which
//                        either scatters q / k / v (q to a buffer, k and v
//                        into the caches at `pos`) or writes a row-major
//                        output.
//   decode_attn_kernel   per (b, h) and chunk of 128 cached keys per wave:
//                        scores, max, exp2 weights, sum and the weighted
//                        value sum; HBM-bound on the cache.  With one chunk
//                        (pos + 1 <= chunk) the block writes the head; with
//                        more, each block leaves fp32 partials and the last
//                        chunk block of the (b, h) to finish merges them
//                        (rescaling by the chunk maxima).
//
// Each kernel's work is one dependent chain of memory accesses (loads, a
// block-local reduction, stores): a decode step is three such launches.
//
// "Last block to finish": each block writes its partials with device-scope
// stores, waits for them, and increments an arrival counter; the block that
// sees the count reach the number of blocks reads every block's partials with
// device-scope loads in a fixed order (deterministic results) and resets the
// counter to zero for the next launch.
#pragma once

#include "common.cuh"

namespace gpt_attn {

constexpr int kDecMaxB = 16;     // rows of one decode call
constexpr int kDecCols = 16;     // output columns per skinny-GEMM block

// Device-scope accesses of the fp32 partials that one block writes and the
// last block of its group reads back.  Relaxed atomics at agent scope are
// plain loads and stores marked coherent across the XCDs' L2 caches, so the
// hand-off needs no whole-cache write-back or invalidation: each thread
// waits until its partial stores have completed (vmcnt(0)) before the block
// barrier that precedes the arrival count, and the last block reads the
// partials with device-scope loads after the count.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0), other counters untouched (gfx9 encoding)
__device__ __forceinline__ void wait_stores() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}
// Arrival count of a block of the group whose counter is *c, out of n
// blocks: true in the block that arrives last (which also resets *c).
__device__ __forceinline__ bool arrive_last(unsigned* c, unsigned n, int* flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == n - 1;
    if (old == n - 1) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *flag != 0;
}

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

// out.put(b, n, sum_c x[b][c] W[c][n] + bias[n]) for b < B (<= kDecMaxB = 16)
// and the block's kDecCols = 16 columns n, on the matrix cores:
// v_mfma_f32_16x16x32_bf16 with A = the W slice transposed (16 columns n x 32
// rows c) and B = x transposed (32 rows c x 16 batch rows b), so that
// D[i][j] = out[j][n0 + i] and the sum over c runs inside the MFMA.  The rows
// go in k-steps of 32; wave w takes the steps w, w + 8, ..., kDecBatchSteps
// at a time, and copies the W rows of those steps (32 B per row: 16 columns)
// into its own LDS slots with global_load_lds_dwordx4 (one 1 KB load per
// step), so it needs no barrier before reading them: lane l of 16-lane group G = l / 16 reads, with
// ds_read_b64_tr_b16, rows 8G + 4t + (l % 16) / 4 (t = 0, 1) at column
// 4 (l % 4) of the step, which hands it the A operand (column l % 16, rows
// 8G .. 8G + 7).  Its B operand, x[b][8G .. 8G + 7] with b = l % 16, is one
// 16-byte load.  The 8 waves' 16 x 16 accumulators are summed in LDS (fixed
// order: deterministic) and the epilogue applied.
constexpr int kDecWaves = 8;
constexpr int kDecBatchSteps = 4;   // k-steps whose x operands are loaded together

__device__ __align__(16) static const uint4 g_dec_zero16 = {0u, 0u, 0u, 0u};

template <class Out>
__global__ __launch_bounds__(64 * kDecWaves) void skinny_gemm_kernel(
    const bf16_t* __restrict__ x, int B, int K, const bf16_t* __restrict__ W, int N,
    const bf16_t* __restrict__ bias, Out out) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  extern __shared__ __align__(16) char dsm[];
  float* red = reinterpret_cast<float*>(dsm);                     // [kDecWaves][64][4]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // this wave's W slots: kDecBatchSteps k-steps of [32 rows][32 B]
  char* wslot = dsm + kDecWaves * 64 * 4 * sizeof(float) + w * kDecBatchSteps * 1024;
  const int n0 = blockIdx.x * kDecCols;
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
                  ? *reinterpret_cast<const bf16x8*>(x + (size_t)bj * K + k)
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
  // lane l holds D[4 (l / 16) + r][l % 16], r = 0..3
  *reinterpret_cast<floatx4*>(red + (w * 64 + lane) * 4) = acc;
  __syncthreads();
  const int o = threadIdx.x;  // output (i, j) = (o / 16, o % 16)
  if (o < 256) {
    const int i = o >> 4, j = o & 15;
    const int l = (i >> 2) * 16 + j, r = i & 3;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) v += red[(ww * 64 + l) * 4 + r];
    const int n = n0 + i;
    if (j < B && n < N) {
      if (bias) v += bf2f(bias[n]);
      out.put(j, n, v);
    }
  }
}

// Attention of one query per (b, h) over cached keys [chunk * CHUNK,
// min(pos + 1, (chunk + 1) * CHUNK)), CHUNK = 128 keys per wave of the NT
// threads.  Each wave takes 128
// consecutive keys and runs on its own as its loads arrive: lane l scores
// keys l and l + 64, the wave takes its max, exp2 weights and sum, passes
// the weights through its own LDS slice, and for the weighted value sum lane
// l takes 8 value columns (dg) of a group of consecutive keys (kg); the
// groups are summed with lane shuffles.  The 8 waves' (m, l, o) then merge
// after the block's one barrier, each rescaled to the common maximum.  One
// chunk: the block writes y_m[b][h*HS + d] = bf16(o / l).  Several: it writes
// (m, l, o[0..HS)) in fp32 (m the chunk's max of the log2-scaled scores,
// l = sum 2^(s - m), o = sum 2^(s - m) v), and the last chunk block of the
// (b, h) to finish merges the chunks the same way.
template <int HS, int NT>
__global__ __launch_bounds__(NT) void decode_attn_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, float* __restrict__ part, bf16_t* __restrict__ ym, int H,
    int cache_T, int pos, int nchunk, float scale_log2, unsigned* __restrict__ counters) {
  constexpr int NW = NT / 64;
  constexpr int KPW = 128;                  // keys per wave
  constexpr int CHUNK = NW * KPW;           // keys per block
  constexpr int DG = HS / 8, KG = 64 / DG;  // value columns / key groups per wave
  constexpr int KPG = KPW / KG;             // keys per group
  __shared__ float ps[NW][KPW];
  __shared__ float wpart[NW][HS + 2];
  __shared__ int is_last;
  const int bh = blockIdx.x, chunk = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int C = H * HS;
  const size_t head = ((size_t)b * H + h) * cache_T * HS;
  const int kw0 = chunk * CHUNK + w * KPW;  // this wave's first key
  const int dg = lane % DG, kg = lane / DG;
  const int jb = kw0 + kg * KPG;
  uint4 vr[KPG];
#pragma unroll
  for (int u = 0; u < KPG; ++u)
    vr[u] = jb + u <= pos
                ? *reinterpret_cast<const uint4*>(v_cache + head + (size_t)(jb + u) * HS + 8 * dg)
                : make_uint4(0u, 0u, 0u, 0u);
  uint4 kr[2][HS / 8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = kw0 + lane + 64 * t;
#pragma unroll
    for (int d8 = 0; d8 < HS / 8; ++d8)
      kr[t][d8] = j <= pos
                      ? *reinterpret_cast<const uint4*>(k_cache + head + (size_t)j * HS + 8 * d8)
                      : make_uint4(0u, 0u, 0u, 0u);
  }
  float s[2];
  float m = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = kw0 + lane + 64 * t;
    float acc = 0.f;
#pragma unroll
    for (int d8 = 0; d8 < HS / 8; ++d8) {
      const uint4 uq = *reinterpret_cast<const uint4*>(q + (size_t)b * C + h * HS + 8 * d8);
      const unsigned wq[4] = {uq.x, uq.y, uq.z, uq.w};
      const unsigned wd[4] = {kr[t][d8].x, kr[t][d8].y, kr[t][d8].z, kr[t][d8].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf2f(wq[e] & 0xffff), bf2f(wd[e] & 0xffff), acc);
        acc = fmaf(bf2f(wq[e] >> 16), bf2f(wd[e] >> 16), acc);
      }
    }
    s[t] = j <= pos ? acc * scale_log2 : -INFINITY;
    m = fmaxf(m, s[t]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  // weights of keys past pos are 0 (also when the whole wave is past pos)
  float l = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float p = kw0 + lane + 64 * t <= pos ? __builtin_amdgcn_exp2f(s[t] - m) : 0.f;
    ps[w][lane + 64 * t] = p;
    l += p;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  // the wave's weights are read back by other lanes of the same wave
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float o8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    const float pj = ps[w][kg * KPG + u];
    const unsigned wd[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o8[2 * e] = fmaf(pj, bf2f(wd[e] & 0xffff), o8[2 * e]);
      o8[2 * e + 1] = fmaf(pj, bf2f(wd[e] >> 16), o8[2 * e + 1]);
    }
  }
  // sum the key groups: lanes dg, dg + DG, ... hold the same columns
#pragma unroll
  for (int o = DG; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] += __shfl_xor(o8[e], o);
  if (kg == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wpart[w][2 + 8 * dg + e] = o8[e];
  }
  if (lane == 0) {
    wpart[w][0] = m;
    wpart[w][1] = l;
  }
  __syncthreads();
  // merge the waves (fixed order)
  float mm = -INFINITY, ll = 0.f, oo = 0.f;
  if (tid < HS) {
#pragma unroll
    for (int i = 0; i < NW; ++i) mm = fmaxf(mm, wpart[i][0]);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const float a = wpart[i][1] > 0.f ? __builtin_amdgcn_exp2f(wpart[i][0] - mm) : 0.f;
      ll = fmaf(wpart[i][1], a, ll);
      oo = fmaf(wpart[i][2 + tid], a, oo);
    }
  }
  if (nchunk == 1) {
    if (tid < HS) ym[(size_t)b * C + h * HS + tid] = f2bf(oo / ll);
    return;
  }
  if (tid < HS) {
    float* pr = part + ((size_t)bh * nchunk + chunk) * (HS + 2);
    st_dev(&pr[2 + tid], oo);
    if (tid == 0) {
      st_dev(&pr[0], mm);
      st_dev(&pr[1], ll);
    }
  }
  // the last chunk block of this (b, h) merges the chunks in order
  if (!arrive_last(&counters[bh], (unsigned)nchunk, &is_last)) return;
  if (tid < HS) {
    const float* pr = part + (size_t)bh * nchunk * (HS + 2);
    float cm = -INFINITY;
    for (int c = 0; c < nchunk; ++c) cm = fmaxf(cm, ld_dev(&pr[c * (HS + 2)]));
    float cl = 0.f, co = 0.f;
    for (int c = 0; c < nchunk; ++c) {
      const float a = __builtin_amdgcn_exp2f(ld_dev(&pr[c * (HS + 2)]) - cm);
      cl = fmaf(ld_dev(&pr[c * (HS + 2) + 1]), a, cl);
      co = fmaf(ld_dev(&pr[c * (HS + 2) + 2 + tid]), a, co);
    }
    ym[(size_t)b * C + h * HS + tid] = f2bf(co / cl);
  }
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
inline size_t skinny_lds_bytes() {
  return (size_t)kDecWaves * 64 * 4 * sizeof(float) + (size_t)kDecWaves * kDecBatchSteps * 1024;
}

}  // namespace gpt_attn
