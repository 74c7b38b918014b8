// common.cuh -- element types, vector types and small device helpers for the
// gfx950 (CDNA4) kernels of the causal self-attention layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt_attn {

typedef uint16_t bf16_t;  // bfloat16 bit pattern as stored in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest even (lowers to v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

__device__ __forceinline__ float bf2f(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Non-temporal 16-byte store, for a call's final outputs (no later kernel of
// the call reads them): the line goes out without staying dirty in the
// XCD's L2, where the next kernel's traffic would otherwise write it back.
__device__ __forceinline__ void store16_stream(void* p, uint4 w) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// 16-byte store written through the XCD's L2 (a buffer store with the sc1
// cache policy), for a tensor that the next kernel reads, largely from other
// XCDs: the line does not stay dirty in this XCD's L2, so no write-back of
// it lands in the next kernel.  base: the tensor; off: byte offset, < 2^31.
__device__ __forceinline__ void store16_wt(void* base, uint32_t off, uint4 w) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {w.x, w.y, w.z, w.w};
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 16 /* sc1 */);
}

// Two fp32 -> packed pair of bf16 (low half = a), round to nearest even as
// f2bf.  Written as one two-lane vector conversion, which is a single
// v_cvt_pk_bf16_f32 (two scalar conversions cost that instruction twice plus
// a shift and an or).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  typedef float float2_v __attribute__((ext_vector_type(2)));
  const bf16x2_v v = __builtin_convertvector((float2_v){a, b}, bf16x2_v);
  return __builtin_bit_cast(uint32_t, v);
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%32][k-slice of
// lane half l/32] and B[k-slice][l%32]; the result tile D has, in lane l,
// column l%32 and rows 8*(r/4) + 4*(l/32) + (r%4) for register r = 0..15.
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace gpt_attn
