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
//   decode_attn_kernel   per (b, h) and chunk of KPW cached keys per wave:
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
#include "skinny.cuh"

namespace gpt_attn {

constexpr int kDecMaxB = 16;     // rows of one decode call

// Device-scope accesses of the fp32 partials that one block writes and the
// last block of its group reads back: relaxed atomics at agent scope, i.e.
// loads and stores coherent across the XCDs' L2 caches.  The ordering of the
// hand-off comes from the arrival count (arrive_last): every thread's partial
// stores precede the block barrier, the barrier precedes thread 0's
// acquire-release increment at agent scope, and in the last block that
// increment precedes the barrier after which its threads load the partials.
// So each block's stores happen before the last block's loads (release
// sequence on the counter, chained with the workgroup barriers).
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
    const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
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
// and the block's kDecCols = 16 columns n (skinny.cuh: the MFMA block).
template <class Out>
__global__ __launch_bounds__(64 * kDecWaves) void skinny_gemm_kernel(
    const bf16_t* __restrict__ x, int B, int K, const bf16_t* __restrict__ W, int N,
    const bf16_t* __restrict__ bias, Out out) {
  extern __shared__ __align__(16) char dsm[];
  const int n0 = blockIdx.x * kDecCols;
  skinny_mfma(x, K, B, K, W, N, n0, dsm);
  const float* red = reinterpret_cast<const float*>(dsm);
  const int o = threadIdx.x;  // output (i, j) = (o / 16, o % 16)
  if (o < 256) {
    const int i = o >> 4, j = o & 15;
    const float v = red[((i >> 2) * 16 + j) * 4 + (i & 3)];
    const int n = n0 + i;
    if (j < B && n < N) out.put(j, n, bias ? v + bf2f(bias[n]) : v);
  }
}

// Attention of one query per (b, h) over cached keys [chunk * CHUNK,
// min(pos + 1, (chunk + 1) * CHUNK)), CHUNK = KPW keys per wave of the NT
// threads.  Each wave takes KPW consecutive keys and runs on its own as its
// loads arrive.  Lane l holds 8 columns (dg = l % (HS/8)) of the key and
// value rows of a group of consecutive keys (kg = l / (HS/8)), so every load
// instruction reads whole 128-byte rows (a lane per 16-byte chunk) for both
// caches.  A key's score is the sum of its group's HS/8 partial dot products
// (lane shuffles inside the group, after which every lane of the group holds
// the group's scores); the wave's max and sum and the weighted value sum are
// then taken over the groups.  The waves' (m, l, o) merge after the block's
// one barrier, each rescaled to the common maximum.  More, shorter waves per
// block keep more of the cache's loads in flight on the block's CU (16 waves
// of 64 keys: a 1024-key cache in one block).  One chunk: the block writes
// y_m[b][h*HS + d] = bf16(o / l).  Several: it writes (m, l, o[0..HS)) in
// fp32 (m the chunk's max of the log2-scaled scores, l = sum 2^(s - m),
// o = sum 2^(s - m) v), and the last chunk block of the (b, h) to finish
// merges the chunks the same way.
template <int HS, int NT, int KPW>
__global__ __launch_bounds__(NT) void decode_attn_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, float* __restrict__ part, bf16_t* __restrict__ ym, int H,
    int cache_T, int pos, int nchunk, float scale_log2, unsigned* __restrict__ counters) {
  constexpr int NW = NT / 64;
  constexpr int CHUNK = NW * KPW;           // keys per block
  constexpr int DG = HS / 8, KG = 64 / DG;  // column chunks of a row / key groups per wave
  constexpr int KPG = KPW / KG;             // keys per group
  static_assert(KPW % KG == 0, "whole key groups per wave");
  __shared__ float wpart[NW][HS + 2];
  __shared__ int is_last;
  const int bh = blockIdx.x, chunk = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int C = H * HS;
  const size_t head = ((size_t)b * H + h) * cache_T * HS;
  const int kw0 = chunk * CHUNK + w * KPW;  // this wave's first key
  const int dg = lane % DG, kg = lane / DG;
  const int jb = kw0 + kg * KPG;            // this group's first key
  uint4 kr[KPG], vr[KPG];
#pragma unroll
  for (int u = 0; u < KPG; ++u)
    kr[u] = jb + u <= pos
                ? *reinterpret_cast<const uint4*>(k_cache + head + (size_t)(jb + u) * HS + 8 * dg)
                : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int u = 0; u < KPG; ++u)
    vr[u] = jb + u <= pos
                ? *reinterpret_cast<const uint4*>(v_cache + head + (size_t)(jb + u) * HS + 8 * dg)
                : make_uint4(0u, 0u, 0u, 0u);
  float qf[8];
  {
    const uint4 uq = *reinterpret_cast<const uint4*>(q + (size_t)b * C + h * HS + 8 * dg);
    const unsigned wq[4] = {uq.x, uq.y, uq.z, uq.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[2 * e] = bf2f(wq[e] & 0xffff);
      qf[2 * e + 1] = bf2f(wq[e] >> 16);
    }
  }
  // partial dot products over this lane's 8 columns, summed over the group
  float s[KPG];
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    const unsigned wd[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(qf[2 * e], bf2f(wd[e] & 0xffff), acc);
      acc = fmaf(qf[2 * e + 1], bf2f(wd[e] >> 16), acc);
    }
    s[u] = acc;
  }
#pragma unroll
  for (int o = 1; o < DG; o <<= 1)
#pragma unroll
    for (int u = 0; u < KPG; ++u) s[u] += __shfl_xor(s[u], o);
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    s[u] = jb + u <= pos ? s[u] * scale_log2 : -INFINITY;
    m = fmaxf(m, s[u]);
  }
#pragma unroll
  for (int o = DG; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  // weights of keys past pos are 0 (also when the whole wave is past pos)
  float l = 0.f;
  float o8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    const float pj = jb + u <= pos ? __builtin_amdgcn_exp2f(s[u] - m) : 0.f;
    l += pj;
    const unsigned wd[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o8[2 * e] = fmaf(pj, bf2f(wd[e] & 0xffff), o8[2 * e]);
      o8[2 * e + 1] = fmaf(pj, bf2f(wd[e] >> 16), o8[2 * e + 1]);
    }
  }
  // sum the key groups: lanes dg, dg + DG, ... hold the same columns
#pragma unroll
  for (int o = DG; o < 64; o <<= 1) {
    l += __shfl_xor(l, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] += __shfl_xor(o8[e], o);
  }
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


}  // namespace gpt_attn
