// philox.cuh -- Philox4x32-10 counter-based generator and the dropout keep
// rule of the layer.
//
// Philox4x32 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): a 4-word counter is mixed with a 2-word key by ten
// rounds; each round multiplies counter words 0 and 2 by two fixed odd
// constants (32 x 32 -> 64 bits), xors the high halves with words 1 and 3
// and the round key, and moves the low halves into words 1 and 3; the key
// advances by two Weyl constants between rounds.
//
// Dropout (nn.Dropout after the softmax and after c_proj; page "nanoGPT
// architecture explained step by step", section 3): kept elements are scaled
// by 1 / (1 - p).  Attention weight (b, h, i, j): counter (j / 8, i, b * H + h,
// 1), 16-bit half j % 2 of word (j % 8) / 2, dropped iff that half is below
// floor(p * 2^16) (one call covers eight keys).  c_proj output (m, n):
// counter (n / 4, m, 0, 2), word n % 4, dropped iff below floor(p * 2^32).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gpt_attn {

struct DropParams {
  uint32_t k0, k1;   // key: seed low / high word
  uint32_t thresh;   // c_proj output: drop iff word < thresh
  uint32_t thresh16; // attention weights: drop iff 16-bit half < thresh16
  float scale;       // 1 / (1 - p)
};

// Each round's products are written as 32 x 32 -> 64-bit multiplies, which
// become one v_mad_u64_u32 per word instead of a separate high and low
// multiply, and each three-way xor is one v_bitop3_b32 (truth table 0x96 =
// a ^ b ^ c): together about 1.6x the calls per second on gfx950, same words.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4(xor3((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1,
                   xor3((uint32_t)(p0 >> 32), c.w, k1), (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

}  // namespace gpt_attn
