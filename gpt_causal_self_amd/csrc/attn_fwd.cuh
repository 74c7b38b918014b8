// attn_fwd.cuh -- fused causal attention forward for gfx950.
//
// Computes, for every (batch b, head h, query i):
//   o_i = sum_{j <= i} softmax_j(q_i . k_j / sqrt(hs)) v_j
// (page "nanoGPT global flow walkthrough", section 2.5 (B), forward steps 3-6:
// scores scaled by 1/sqrt(hs), tril mask to -inf, row softmax, att @ v) and
// writes o straight into the merged-head layout y_m[b][i][h*hs + d] (step 7's
// transpose + view), never materialising the T x T score matrix.
//
// bf16 kernel (MFMA).  One block = 4 waves = 128 queries of one (b, h); each
// wave owns 32 queries.  Keys and values are streamed through an LDS ring in
// tiles of 64 (the next tiles' global loads are in flight during the current
// tile's math).  Per tile a wave computes S^T = K Q^T (keys on the
// MFMA rows, its 32 queries on the columns) with 32x32x16 bf16 MFMAs, so each
// lane holds 32 scores of ONE query: the row max / row sum of the online
// softmax are a local reduction plus one exchange with the other lane half.
// The probabilities, rounded to bf16, are already laid out as the B operand
// of O^T += V^T P^T; the V^T operand is read from a transposed LDS copy of the
// value tile with the matching key order.  Softmax statistics are fp32 in the
// exp2 domain (scale * log2(e) folded into one multiply).  Tiles entirely above
// the diagonal are never loaded; a wave skips a tile that lies entirely in
// its future; diagonal tiles are masked in place.  Heavier (later) query
// tiles are dispatched first.
//
// fp32 kernel (FMA).  One wave of 64 threads per 64 queries, one query per
// thread, key/value tiles in LDS, online softmax key by key.
#pragma once

#include <type_traits>

#include "common.cuh"
#include "gemm2.cuh"
#include "keep_bits.cuh"
#include "philox.cuh"

namespace gpt_attn {

constexpr int kAttnBQ = 128;  // queries per block (bf16 kernel)
constexpr int kAttnBK = 64;   // keys per tile

// Reductions over the lane pairs (l, l ^ 32) of a wave with
// v_permlane32_swap: the swap of a value with itself hands every lane both
// x[l % 32] and x[l % 32 + 32], so the pair's max or sum needs no LDS
// round trip (a __shfl_xor goes through ds_bpermute).  Both lanes of a pair
// get the same value, formed in the same order.
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource of a bf16 slab of n_bytes bytes at p: raw (stride 0)
// addressing, 32-bit data format; loads at byte offsets at or beyond
// n_bytes return zeros, which is how a tile that crosses the sequence end
// reads its missing rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* p, uint32_t n_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n_bytes,
                                           0x00020000);
}
// 16 bytes per lane from the slab at voffset + soffset (bytes) straight into
// LDS at lds (+ 16 * lane).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds,
                                                uint32_t voffset, uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, soffset, 0, 0);
}


// ----------------------------------------------------- bf16, pipelined
// Details of the bf16 kernel:
//  * K and V tiles moved global -> LDS by global_load_lds_dwordx4 into an
//    NS-stage ring (manual vmcnt waits, bare barriers), rows of hs elements
//    with 16-byte chunks XOR-swizzled by the key row;
//  * the V^T MFMA operand read with ds_read_b64_tr_b16 straight from the
//    [key][d] tile, in the permuted key order of the probability registers
//    (no register transposition);
//  * the score scale folded into the exp2 argument with one FMA, and lazy
//    rescaling: the running reference (a whole number in log2 units, at or
//    above the max that set it) only moves (rescaling l and the accumulators)
//    when a tile's max exceeds it by more than 8, so unnormalised weights
//    stay below 2^8 and most tiles skip the rescale.  Each weight is rounded
//    to bf16 as the P.V operand; the row sum adds the unrounded weights.
// Chunk swizzle of a key row.  LDS has 64 four-byte banks (256 bytes per
// bank line), so a 128-byte row (HS = 64) shares its bank line with one
// neighbour and a 64-byte row (HS = 32) with three.  The swizzle keeps both
// read patterns conflict-free:
//  * b128 fragment reads: 16 lanes read one chunk of 16 consecutive rows;
//    rows of the same bank-line position must use distinct chunks, so the
//    swizzle runs over bits 1..3 (HS = 64) or 2..3 (HS = 32) of the row;
//  * transposing reads: 32 lanes read chunks 0..3 (or 4..7) of 4
//    consecutive rows 4a..4a+3; for HS = 64 rows 4a and 4a+2 must land in
//    different chunk halves, so bit 1 of the row moves the chunk by 4.
// The swizzle depends on bits 1..3 of the row only: it repeats every 16 rows.
template <int HS>
__device__ __forceinline__ int kv_swz(int row) {
  return HS == 64 ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)) : ((row >> 2) & 3);
}

// Offset of a transposing read 8t rows below the one at offset `off`
// (t = 0, 1): for both head sizes kv_swz(r + 8) = kv_swz(r) ^ 2, i.e. chunk
// bit 1 (offset bit 5) flips; rows are RB bytes apart.
template <int RB>
__device__ __forceinline__ int tr_off(int off, int t) {
  return t ? ((off ^ 32) + 8 * RB) : off;
}

// DROP: dropout on the attention weights (philox.cuh): the row sum uses
// every weight, the P.V product only the kept ones, and the output is scaled
// by 1 / (1 - p).  With keepq / keepk (a forward whose state the backward
// uses) the keep decisions are also stored, one bit per weight, in the two
// layouts of keep_bits.cuh, so that the backward reads them instead of
// drawing the generator again.
template <int HS, int NS, bool DROP = false>
__global__ __launch_bounds__(256, 2) void attn_fwd2_bf16_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kg,
    const bf16_t* __restrict__ Vg, bf16_t* __restrict__ O, float* __restrict__ lse,
    int H, int T, float scale_log2, DropParams drop = {}, uint32_t* __restrict__ keepq = nullptr,
    uint16_t* __restrict__ keepk = nullptr) {
  static_assert(HS == 32 || HS == 64, "head size");
  constexpr int BKV = kAttnBK;
  constexpr int TILE = BKV * HS * 2;   // bytes of one K or V tile
  constexpr int STAGE = 2 * TILE;
  constexpr int RB = HS * 2;           // bytes of one key row
  constexpr int CPR = HS / 8;          // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;        // key rows per 1 KB load
  constexpr int LPW = TILE / 1024 / 4; // loads per wave per tile (K or V)
  constexpr int kLoads = 2 * LPW;
  constexpr float kLazy = 8.f;         // rescale threshold (log2 units)
  __shared__ __align__(1024) char smem[NS * STAGE];

  const int nqt = (T + kAttnBQ - 1) / kAttnBQ;
  const int bh = blockIdx.x;
  const int qt = nqt - 1 - (int)blockIdx.y;  // heavy tiles first
  const int b = bh / H, h = bh - b * H;
  const size_t head = (size_t)bh * T * HS;
  const bf16_t* Qh = Q + head;
  const bf16_t* Kh = Kg + head;
  const bf16_t* Vh = Vg + head;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int hi = lane >> 5;
  const int q0 = qt * kAttnBQ + wid * 32;
  const int myq = q0 + (lane & 31);

  bf16x8 qf[HS / 16];
#pragma unroll
  for (int kk = 0; kk < HS / 16; ++kk)
    qf[kk] = myq < T ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)myq * HS + 16 * kk + 8 * hi)
                     : bf16x8{};
  floatx16 acc[HS / 32];
#pragma unroll
  for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  // Loop-invariant LDS offsets.  K fragment (row kt*32 + lane%32, chunk
  // 2kk + hi): rows differ from lane%32 by multiples of 32, which leave the
  // swizzle unchanged, so only kk and the lane matter.  V transposing reads
  // (row kb + 8t + 4(G/2) + s/4, column dt*32 + 16(G%2) + 4(s%4)): kb is a
  // multiple of 16, so the swizzle depends on t and the lane part r0 only.
  int koff[HS / 16];
#pragma unroll
  for (int kk = 0; kk < HS / 16; ++kk) {
    const int row = lane & 31;
    koff[kk] = row * RB + (((2 * kk + hi) ^ kv_swz<HS>(row)) << 4);
  }
  const int G = lane >> 4, s16 = lane & 15;
  const int r0 = 4 * (G >> 1) + (s16 >> 2);
  int voff[2][HS / 32];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int dt = 0; dt < HS / 32; ++dt) {
      const int d = dt * 32 + 16 * (G & 1) + 4 * (s16 & 3);
      const int r = r0 + 8 * t;
      voff[t][dt] = r * RB + (((d >> 3) ^ kv_swz<HS>(r)) << 4) + ((d >> 2) & 1) * 8;
    }

  const int kv_end = min(T, (qt + 1) * kAttnBQ);
  const int nkv = (kv_end + BKV - 1) / BKV;

  // Loads of the K and V tile starting at key j0 into the ring stage at dst,
  // through buffer resources over the (b, h) slabs of K and V: the per-lane
  // byte offset within a tile is loop-invariant (lane -> (row, chunk) of
  // load q), the tile's start j0 * HS * 2 is a wave-uniform offset, and
  // rows past T lie beyond the slab and read zeros.
  const __amdgpu_buffer_rsrc_t rk = slab_rsrc(Kh, (uint32_t)T * HS * 2);
  const __amdgpu_buffer_rsrc_t rv = slab_rsrc(Vh, (uint32_t)T * HS * 2);
  uint32_t src_off[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int row = (wid * LPW + q) * RPI + lane / CPR;
    src_off[q] = (uint32_t)(row * HS + ((lane % CPR) ^ kv_swz<HS>(row)) * 8) * 2;
  }
  auto issue = [&](char* dst, int j0) {
    const uint32_t so = (uint32_t)j0 * HS * 2;
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      char* base = dst + (wid * LPW + q) * 1024;
      buffer_to_lds16(rk, base, src_off[q], so);
      buffer_to_lds16(rv, base + TILE, src_off[q], so);
    }
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nkv) issue(smem + s * STAGE, s * BKV);

  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) const bf16x8 lds_b128;

  // Keep bits of the last tile this wave computed, stored at the start of the
  // next tile (before its ring loads, so the ring's vmcnt waits find them
  // long complete) or after the loop.
  const KeepBitsLayout kl(T);
  const bool store_keep = DROP && keepq != nullptr;
  uint32_t pend_q = 0, pend_k = 0;
  int pend_jt = -1;
  auto flush_keep = [&]() {
    if (store_keep && pend_jt >= 0) {
      keepq[kl.q_index(bh, pend_jt, hi, myq)] = pend_q;
      const size_t k0 = kl.k_index(bh, q0 >> 6, 0, pend_jt * 64 + lane);
      const int qh = (q0 >> 5) & 1;
      keepk[2 * k0 + qh] = (uint16_t)pend_k;
      keepk[2 * (k0 + kl.Tk) + qh] = (uint16_t)(pend_k >> 16);
      pend_jt = -1;
    }
  };

  // One 64-key tile held in ring stage rd; first issues the loads of the tile
  // at key jn into stage wr (when jn >= 0).  MASK: apply the causal mask
  // (diagonal tiles).  rd and wr are distinct stages: the restrict qualifiers
  // tell the compiler so, and it then does not make the reads of rd wait for
  // the loads into wr (the ring's vmcnt waits and barriers order them).
  auto tile = [&](auto mask_tag, const char* __restrict__ rd, char* __restrict__ wr, int jn,
                  int j0) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (DROP) flush_keep();
    if (jn >= 0) issue(wr, jn);
    const lds_char* lbase = (const lds_char*)rd;
    // ---- S^T = K Q^T for keys j0 .. j0+63
    floatx16 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kt][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < HS / 16; ++kk) {
        const bf16x8 kf = *(lds_b128*)(lbase + koff[kk] + kt * 32 * RB);
        sc[kt] = mfma32(kf, qf[kk], sc[kt]);
      }
    }
    if constexpr (MASK) {
      // key - myq = (j0 - q0) + kt*32 + 8(r/4) + 4hi + r%4 - lane%32
      const int lim = myq - j0 - 4 * hi;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + 8 * (r >> 2) + (r & 3) > lim) sc[kt][r] = -INFINITY;
    }
    float smax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sc[kt][r]);
    smax = pair_max32(smax);
    const float tmax = smax * scale_log2;
    // ---- lazy rescale (wave-uniform branch).  The reference is a whole
    // number (log2 units), so every weight is the true softmax weight times a
    // power of two: its bf16 rounding below does not depend on which tile
    // last moved the reference.
    const bool need = tmax > m + kLazy;
    if (__any(need)) {
      const float m_new = need ? __builtin_ceilf(tmax) : m;
      const float alpha = need ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
    // ---- probabilities (relative to m, at most 2^8), row sum
    const float negm = -m;
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[kt][r], scale_log2, negm));
        sc[kt][r] = p;
        rs += p;
      }
    rs = pair_sum32(rs);
    l += rs;
    if constexpr (DROP) {
      // keys j0 + kt*32 + 8g + 4hi + e (e = 0..3) of query myq.  The eight
      // keys j0 + kt*32 + 8g + (0..7) share one Philox call whose 16-bit
      // halves are their draws: lanes l and l + 32 (same query) split the
      // two calls of group g (lane hi draws kt = hi), each keeps the two
      // words of its own four keys and hands the other two to its partner
      // with v_permlane32_swap (r[0] = x[l % 32], r[1] = x[l % 32 + 32]).
      // wq: this lane's keep bits (bit 16kt + 4g + e).
      uint32_t wq = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t jc = (uint32_t)(j0 + hi * 32 + 8 * g) >> 3;
        const uint4 c = philox4x32_10(make_uint4(jc, (uint32_t)myq, (uint32_t)bh, 1u), drop.k0,
                                      drop.k1);
        const uint32_t own0 = hi ? c.z : c.x, own1 = hi ? c.w : c.y;
        const uint32_t sx = hi ? c.x : c.z, sy = hi ? c.y : c.w;
        const auto rx = __builtin_amdgcn_permlane32_swap(sx, sx, false, false);
        const auto ry = __builtin_amdgcn_permlane32_swap(sy, sy, false, false);
        const uint32_t got0 = hi ? rx[0] : rx[1], got1 = hi ? ry[0] : ry[1];
        // words of kt = 0 and kt = 1 for this lane's four keys
        const uint32_t wd[2][2] = {{hi ? got0 : own0, hi ? got1 : own1},
                                   {hi ? own0 : got0, hi ? own1 : got1}};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t u = (wd[kt][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            const bool kp = u >= drop.thresh16;
            if (!kp) sc[kt][4 * g + e] = 0.f;
            wq |= (uint32_t)kp << (16 * kt + 4 * g + e);
          }
      }
      if (store_keep) {
        // lane o: keep bits of key j0 + o over the wave's 32 queries
        const uint32_t xk = keep_transpose(wq);
        pend_q = wq;
        pend_k = keep_half16(xk) | (keep_half16(xk >> 4) << 16);
        pend_jt = j0 >> 6;
      }
    }
    // ---- O^T += V^T P^T; V^T operand by transposing reads in the key order
    // of the P registers: element e <-> key kb + 8(e/4) + 4*hi + e%4.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (__bf16)sc[kt][8 * u + e];
        const int kb = kt * 32 + 16 * u;
#pragma unroll
        for (int dt = 0; dt < HS / 32; ++dt) {
          v4i16 rv[2];
#pragma unroll
          for (int t = 0; t < 2; ++t)
            rv[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(lbase + TILE + voff[t][dt] + kb * RB));
          typedef short v8i16 __attribute__((ext_vector_type(8)));
          const v8i16 vv = {rv[0][0], rv[0][1], rv[0][2], rv[0][3],
                            rv[1][0], rv[1][1], rv[1][2], rv[1][3]};
          acc[dt] = mfma32(__builtin_bit_cast(bf16x8, vv), pf, acc[dt]);
        }
      }
  };

  // Ring step: wait for tile `it` and publish it; returns the first key of
  // the tile whose loads refill the ring (-1: none left).
  auto step = [&](int it) {
    const int later = min(nkv - 1, it + NS - 2) - it;
    if (later >= NS - 2) wait_vmcnt<kLoads * (NS - 2)>();
    else if (NS > 3 && later == 2) wait_vmcnt<kLoads * 2>();
    else if (later == 1) wait_vmcnt<kLoads>();
    else wait_vmcnt<0>();
    bar_nofence();
    return it + NS - 1 < nkv ? (it + NS - 1) * BKV : -1;
  };
  // Tiles wholly below the block's first query need no mask for any wave;
  // the last (at most two) tiles reach the diagonal.
  const int n_full = min(nkv, (qt * kAttnBQ) / BKV);
  int it = 0;
  for (; it < n_full; ++it) {
    const int jn = step(it);
    tile(std::integral_constant<bool, false>{}, smem + (it % NS) * STAGE,
         smem + ((it + NS - 1) % NS) * STAGE, jn, it * BKV);
  }
  for (; it < nkv; ++it) {
    const int jn = step(it);
    const int j0 = it * BKV;
    char* wr = smem + ((it + NS - 1) % NS) * STAGE;
    if (j0 <= q0 + 31)  // skip tiles wholly in this wave's future
      tile(std::integral_constant<bool, true>{}, smem + (it % NS) * STAGE, wr, jn, j0);
    else if (jn >= 0)
      issue(wr, jn);
  }

  if constexpr (DROP) flush_keep();

  if (myq < T) {
    const float inv = (DROP ? drop.scale : 1.f) / l;
    const int C = HS * H;
    bf16_t* orow = O + ((size_t)b * T + myq) * C + h * HS;
#pragma unroll
    for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        uint2 w;
        w.x = pack_bf16x2(acc[dt][4 * g + 0] * inv, acc[dt][4 * g + 1] * inv);
        w.y = pack_bf16x2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
    if (lse != nullptr && hi == 0)
      lse[(size_t)bh * T + myq] = (m + __log2f(l)) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------- fp32
// fp32 path: 64 queries per block, four lanes per query (lane t of a quad
// holds dimensions [t*HS/4, (t+1)*HS/4) of q and of the output); 64-key
// K/V tiles in LDS.  Keys go in chunks of 8: the quad's partial dot
// products meet through two DPP exchanges (all four lanes then hold the same
// scores), and the online softmax rescales once per chunk.
template <int HS>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ Kg, const float* __restrict__ Vg,
    float* __restrict__ O, float* __restrict__ lse, int H, int T, float scale_log2) {
  constexpr int BQ = 64, BKV = 64, D4 = HS / 4, CH = 8;
  __shared__ __align__(16) float Ks[BKV][HS];
  __shared__ __align__(16) float Vs[BKV][HS];
  const int bh = blockIdx.x;
  const int nqt = (T + BQ - 1) / BQ;
  const int qt = nqt - 1 - (int)blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const size_t head = (size_t)bh * T * HS;
  const int tid = threadIdx.x, sub = tid & 3;
  const int myq = qt * BQ + (tid >> 2);
  float q[D4], o[D4];
#pragma unroll
  for (int d = 0; d < D4; d += 4) {
    const float4 v = myq < T ? *reinterpret_cast<const float4*>(Q + head + (size_t)myq * HS +
                                                                sub * D4 + d)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    q[d] = v.x; q[d + 1] = v.y; q[d + 2] = v.z; q[d + 3] = v.w;
    o[d] = o[d + 1] = o[d + 2] = o[d + 3] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = min(T, (qt + 1) * BQ);
  for (int j0 = 0; j0 < kv_end; j0 += BKV) {
    __syncthreads();
    for (int e = tid; e < BKV * HS / 4; e += 256) {
      const int key = e / (HS / 4), d = (e % (HS / 4)) * 4;
      const bool ok = j0 + key < T;
      const size_t g = head + (size_t)(j0 + key) * HS + d;
      *reinterpret_cast<float4*>(&Ks[key][d]) =
          ok ? *reinterpret_cast<const float4*>(Kg + g) : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(&Vs[key][d]) =
          ok ? *reinterpret_cast<const float4*>(Vg + g) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    // keys j0 .. j0+jmax-1 are visible to this query (same for the quad)
    const int jmax = max(0, min(BKV, min(kv_end, myq + 1) - j0));
    for (int c0 = 0; c0 < jmax; c0 += CH) {
      float t[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const float* kr = &Ks[c0 + k][sub * D4];
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D4; ++d) dot = fmaf(q[d], kr[d], dot);
        dot += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dot), 0xB1, 0xF, 0xF, false));
        dot += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dot), 0x4E, 0xF, 0xF, false));
        t[k] = c0 + k < jmax ? dot * scale_log2 : -INFINITY;
      }
      float cmax = t[0];
#pragma unroll
      for (int k = 1; k < CH; ++k) cmax = fmaxf(cmax, t[k]);
      const float m_new = fmaxf(m, cmax);  // finite: key c0 is visible
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D4; ++d) o[d] *= alpha;
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const float p = c0 + k < jmax ? __builtin_amdgcn_exp2f(t[k] - m_new) : 0.f;
        l += p;
        const float* vr = &Vs[c0 + k][sub * D4];
#pragma unroll
        for (int d = 0; d < D4; ++d) o[d] = fmaf(p, vr[d], o[d]);
      }
      m = m_new;
    }
  }
  if (myq < T) {
    const int C = HS * H;
    const float inv = 1.f / l;
    float* orow = O + ((size_t)b * T + myq) * C + h * HS + sub * D4;
#pragma unroll
    for (int d = 0; d < D4; d += 4)
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
    if (lse != nullptr && sub == 0)
      lse[(size_t)bh * T + myq] = (m + __log2f(l)) * 0.69314718055994530942f;
  }
}

}  // namespace gpt_attn
