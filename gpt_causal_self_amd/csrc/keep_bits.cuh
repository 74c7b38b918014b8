// keep_bits.cuh -- stored keep decisions of the attention-weight dropout.
//
// A forward that keeps state for the backward stores, besides drawing the
// dropout of the attention weights (philox.cuh), one bit per weight: bit set
// = kept.  Two layouts, one per backward kernel, each a 32-bit word per lane
// and tile in that kernel's own register order, so a lane reads one word per
// tile with coalesced loads:
//   query-major (dQ kernel, lane = query): word q_index(bh, jt, hi, i) holds
//     the weights (i, j0 + 32kt + 8g + 4hi + e) of the 64-key tile j0 = 64 jt,
//     as bit 16kt + 4g + e;
//   key-major (dK/dV kernel, lane = key): word k_index(bh, it, hi, j) holds
//     the weights (i0 + 32qh + 8g + 4hi + e, j) of the 64-query tile
//     i0 = 64 it, as bit 16qh + 4g + e; its two 16-bit halves (qh = 0, 1)
//     come from two different waves of the forward, which store them as
//     halves.
// Rows are padded: queries and keys to multiples of 128 (the blocks of the
// forward and of the dK/dV kernel), key tiles to ceil(T / 64).  Words of tiles
// wholly above the diagonal are never written nor read; the bits of masked
// weights inside diagonal tiles are written but never used.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gpt_attn {

struct KeepBitsLayout {
  int NKT;  // 64-key tiles
  int Tq;   // query rows, padded to 128
  int Tk;   // key rows, padded to 128
  int NQ64; // 64-query tiles of the padded rows
  __host__ __device__ explicit KeepBitsLayout(int T)
      : NKT((T + 63) / 64), Tq((T + 127) / 128 * 128), Tk((T + 127) / 128 * 128),
        NQ64((T + 127) / 128 * 2) {}
  __host__ __device__ size_t q_index(int bh, int jt, int hi, int i) const {
    return ((size_t)(bh * NKT + jt) * 2 + hi) * Tq + i;
  }
  __host__ __device__ size_t k_index(int bh, int it, int hi, int j) const {
    return ((size_t)(bh * NQ64 + it) * 2 + hi) * Tk + j;
  }
  // words of each layout for BH = B * n_head heads
  __host__ __device__ size_t q_words(int BH) const { return (size_t)BH * NKT * 2 * Tq; }
  __host__ __device__ size_t k_words(int BH) const { return (size_t)BH * NQ64 * 2 * Tk; }
};

// Returns v with lane L replaced by the wave-uniform value lo and lane L + 4
// by hi (v_writelane_b32, lanes as inline constants: one SGPR operand each,
// the constant-bus limit of gfx9 VOP3).  lo and hi are written by the ballot's
// VALU compare just before; the compiler does not guard inline asm against
// that hazard (a write lane read the SGPR's previous value when it followed
// the compare directly), so s_nop 4 gives the five wait states first.
template <int L>
__device__ __forceinline__ uint32_t write_lane_pair(uint32_t v, uint32_t lo, uint32_t hi) {
  static_assert(L >= 0 && L + 4 < 64, "lane");
  asm volatile("s_nop 4\n\tv_writelane_b32 %0, %1, %3\n\tv_writelane_b32 %0, %2, %4"
               : "+v"(v)
               : "s"(lo), "s"(hi), "n"(L), "n"(L + 4));
  return v;
}

// In-wave transpose of the forward's keep bits.  wq: lane L (query
// q0 + L % 32, hi = L / 32) holds the keep bit of key j0 + 32kt + 8g + 4hi + e
// at bit S = 16kt + 4g + e.  The ballot of bit S over the wave has the keys
// j0 + 32kt + 8g + e (lanes 0..31, low word) and j0 + 32kt + 8g + 4 + e (lanes
// 32..63, high word), bit t = query q0 + t; the low word goes to lane
// 32kt + 8g + e, the high word to that lane + 4.  Returns, in lane o, the
// keep bits of key j0 + o over the 32 queries.  All lanes must be active.
template <int S = 0>
__device__ __forceinline__ uint32_t keep_transpose(uint32_t wq, uint32_t xk = 0u) {
  if constexpr (S < 32) {
    const uint64_t bal = __builtin_amdgcn_ballot_w64(((wq >> S) & 1u) != 0u);
    constexpr int L = 32 * (S >> 4) + 8 * ((S >> 2) & 3) + (S & 3);
    xk = write_lane_pair<L>(xk, (uint32_t)bal, (uint32_t)(bal >> 32));
    return keep_transpose<S + 1>(wq, xk);
  } else {
    return xk;
  }
}

// x: keep bits of one key over 32 consecutive queries (bit t = query t).
// Returns the 16 bits of queries 8g + e (g, e = 0..3) as bit 4g + e: the low
// nibble of each byte, packed.
__device__ __forceinline__ uint32_t keep_half16(uint32_t x) {
  x &= 0x0F0F0F0Fu;
  x = (x | (x >> 4)) & 0x00FF00FFu;
  return (x | (x >> 8)) & 0xFFFFu;
}

}  // namespace gpt_attn
