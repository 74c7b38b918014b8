// attn_bwd2.cuh -- pipelined bf16 backward of the fused causal attention.
//
// Same gradient as attn_bwd.cuh (D_i = dO_i . o_i, P recomputed from the
// log-sum-exp, dS = P (dP - D), dq_i = (1/sqrt(hs)) sum_j dS_ij k_j,
// dk_j = (1/sqrt(hs)) sum_i dS_ij q_i, dv_j = sum_i p_ij dO_i; page "nanoGPT
// global flow walkthrough", section 2.5 (B), differentiated by the chain
// rule), organised like the forward kernel:
//  * the tiles that stream (K and V for dQ; Q, dO and the rows' log-sum-exp
//    and D for dK/dV) move global -> LDS with global_load_lds_dwordx4 into a
//    two-stage ring, 16-byte chunks of each row XOR-swizzled by the row;
//  * the operands that need the streamed tile transposed (K^T for dQ; Q^T
//    and dO^T for dK/dV) are read with ds_read_b64_tr_b16 straight from the
//    [row][d] tile, in the permuted row order of the probability registers;
//  * the per-step body takes the stage it reads and the stage it fills as
//    restrict pointers, so the LDS reads never wait for the loads in flight.
// Every output element is written by exactly one lane (dQ: one block per
// 128 queries; dK, dV: one block per 128 keys): no atomics, deterministic.
#pragma once

#include "attn_fwd.cuh"
#include "common.cuh"
#include "gemm2.cuh"
#include "keep_bits.cuh"
#include "philox.cuh"

namespace gpt_attn {

constexpr float kLog2eB = 1.4426950408889634f;

// Epilogue of the c_proj input-gradient GEMM dO = dY W_proj^T that also
// produces the softmax backward row statistics, so dO is not read back:
// D[b,h,t] = sum_d dO[b,t,h,d] O[b,t,h,d] over the bf16 dO just rounded and
// the stored forward output O (fmaf over the 8 values of a 16-byte chunk,
// then a sum of the HS/8 chunks of a head across the lanes that hold them),
// and L[b,h,t] = lse * log2(e), both in rows of Tpad = T rounded up to 64
// (the dK/dV kernel reads whole 64-row tiles; rows past T are never used,
// their lanes select 0).  The GEMM's staged store loop hands consecutive
// 16-byte chunks of a row to consecutive lanes, so the HS/8 lanes of an
// aligned group hold one head.
template <int HS>
struct Epi2DgradRowStats {
  bf16_t* out;         // dO [M][ldc]
  int ldc;             // C
  const bf16_t* bias;  // NULL (no bias on this product)
  const bf16_t* O;     // forward attention output [M][ldc]
  const float* lse;    // [B*H][T]
  float* Dpad;         // [B*H][Tpad]
  float* Lpad;         // [B*H][Tpad]
  int T, H, Tpad;
  static constexpr bool kStaged = true;
  static constexpr bool kStore8All = true;
  __device__ __forceinline__ const bf16_t* bias_ptr() const { return bias; }
  // O's chunk and the row's log-sum-exp, loaded ahead of the stores
  struct Extra {
    uint4 o;
    float lse;
  };
  __device__ __forceinline__ Extra extra(int m, int n, bool ok) const {
    Extra e{make_uint4(0u, 0u, 0u, 0u), 0.f};
    if (ok) {
      e.o = *reinterpret_cast<const uint4*>(O + (size_t)m * ldc + n);
      const int b = m / T, t = m - b * T, h = n / HS;
      e.lse = lse[((size_t)b * H + h) * T + t];
    }
    return e;
  }
  __device__ __forceinline__ void store8_all(int m, int n, uint4 w, bool ok, int lane,
                                             const Extra& ex) const {
    float s = 0.f;
    if (ok) {
      *reinterpret_cast<uint4*>(out + (size_t)m * ldc + n) = w;
      const uint4 o = ex.o;
      const unsigned wa[4] = {w.x, w.y, w.z, w.w}, wo[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fmaf(bf2f(wa[e] & 0xffff), bf2f(wo[e] & 0xffff), s);
        s = fmaf(bf2f(wa[e] >> 16), bf2f(wo[e] >> 16), s);
      }
    }
    s = lane_group_sum<HS / 8>(s);
    if (ok && (lane & (HS / 8 - 1)) == 0) {
      const int b = m / T, t = m - b * T, h = n / HS;
      const size_t bh = (size_t)b * H + h;
      Dpad[bh * Tpad + t] = s;
      Lpad[bh * Tpad + t] = ex.lse * kLog2eB;
    }
  }
};

// ---------------------------------------------------------------- dQ
// One block = 4 waves = 128 queries of one (b, h); wave w owns 32 queries
// (lane = query) and keeps q and dO of its query as MFMA B operands.  Per
// 64-key tile: S^T = K Q^T and dP^T = V dO^T (keys on the MFMA rows),
// P^T = exp2(S^T * scale * log2 e - L), dS^T = P^T (dP^T - D) (with DROP,
// dP carries the keep factor z of the weight, read from the forward's keep
// bits, query-major layout of keep_bits.cuh), dQ^T += K^T dS^T.
template <int HS, bool DROP>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq2_bf16_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg,
    const bf16_t* __restrict__ Vg, const bf16_t* __restrict__ dOg,
    const float* __restrict__ Lpad, const float* __restrict__ Dpad, bf16_t* __restrict__ dqkv,
    int H, int T, int Tpad, float scale, float scale_log2, DropParams drop,
    const uint32_t* __restrict__ keepq) {
  static_assert(HS == 32 || HS == 64, "head size");
  constexpr int BKV = 64;
  constexpr int TILE = BKV * HS * 2;   // bytes of one K or V tile
  constexpr int STAGE = 2 * TILE;
  constexpr int RB = HS * 2;
  constexpr int CPR = HS / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int LPW = TILE / 1024 / 4;
  __shared__ __align__(1024) char smem[2 * STAGE];

  const int nqt = (T + 127) / 128;
  const int bh = blockIdx.x;
  const int qt = nqt - 1 - (int)blockIdx.y;  // heavy tiles first
  const int b = bh / H, h = bh - b * H;
  const int C = H * HS;
  const size_t head = (size_t)bh * T * HS;
  const bf16_t* Kh = Kg + head;
  const bf16_t* Vh = Vg + head;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;
  const int q0 = qt * 128 + wid * 32;
  const int myq = q0 + (lane & 31);

  bf16x8 qf[HS / 16], gf[HS / 16];
#pragma unroll
  for (int kk = 0; kk < HS / 16; ++kk) {
    if (myq < T) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(Qg + head + (size_t)myq * HS + 16 * kk + 8 * hi);
      gf[kk] = *reinterpret_cast<const bf16x8*>(dOg + ((size_t)b * T + myq) * C + h * HS +
                                                16 * kk + 8 * hi);
    } else {
      qf[kk] = bf16x8{};
      gf[kk] = bf16x8{};
    }
  }
  const float L2 = myq < T ? Lpad[(size_t)bh * Tpad + myq] : 0.f;
  const float Dq = myq < T ? Dpad[(size_t)bh * Tpad + myq] : 0.f;
  floatx16 dq[HS / 32];
#pragma unroll
  for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  // LDS offsets: row fragments (row kt*32 + lane%32, chunk 2kk + hi) and the
  // transposing reads (row kb + 8t + 4(G/2) + s/4, column dt*32 + 16(G%2) +
  // 4(s%4)), as in the forward kernel.
  int koff[HS / 16];
#pragma unroll
  for (int kk = 0; kk < HS / 16; ++kk) {
    const int row = lane & 31;
    koff[kk] = row * RB + (((2 * kk + hi) ^ kv_swz<HS>(row)) << 4);
  }
  const int G = lane >> 4, s16 = lane & 15;
  const int r0 = 4 * (G >> 1) + (s16 >> 2);
  // t = 1 (rows r0 + 8) flips chunk bit 1 of the swizzle: offset bit 5.
  int toff[HS / 32];
#pragma unroll
  for (int dt = 0; dt < HS / 32; ++dt) {
    const int d = dt * 32 + 16 * (G & 1) + 4 * (s16 & 3);
    toff[dt] = r0 * RB + (((d >> 3) ^ kv_swz<HS>(r0)) << 4) + ((d >> 2) & 1) * 8;
  }

  const int kv_end = min(T, (qt + 1) * 128);
  const int nkv = (kv_end + BKV - 1) / BKV;

  // Loop-invariant per-lane byte offsets within a tile, loads through buffer
  // resources over the (b, h) slabs of K and V: a tile at key j0 adds the
  // wave-uniform j0 * HS * 2, and rows past T read zeros.
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
  issue(smem, 0);

  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) const bf16x8 lds_b128;

  // kw: this lane's keep bits of the tile (bit 16kt + 4g + e)
  auto tile = [&](auto mask_tag, const char* __restrict__ rd, char* __restrict__ wr, int jn,
                  int j0, uint32_t kw) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (jn >= 0) issue(wr, jn);
    const lds_char* lbase = (const lds_char*)rd;
    // one 32-key half at a time: its scores, softmax gradient and dQ product
    // (half the score registers live, for three waves per SIMD)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      floatx16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < HS / 16; ++kk) {
        const bf16x8 kf = *(lds_b128*)(lbase + koff[kk] + kt * 32 * RB);
        const bf16x8 vf = *(lds_b128*)(lbase + TILE + koff[kk] + kt * 32 * RB);
        sc = mfma32(kf, qf[kk], sc);
        dp = mfma32(vf, gf[kk], dp);
      }
      // lane = query myq; register r <-> key j0 + kt*32 + 8(r/4) + 4hi + r%4
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, -L2));
          float dpv = dp[r];
          if constexpr (DROP) dpv *= ((kw >> (16 * kt + r)) & 1u) ? drop.scale : 0.f;
          float ds = p * (dpv - Dq);
          if constexpr (MASK) {
            const int key = j0 + kt * 32 + 8 * g + 4 * hi + e;
            if (key > myq) ds = 0.f;
          }
          dp[r] = ds;
        }
      }
      // dQ^T += K^T dS^T; K^T by transposing reads in the key order of dS
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 sf;
#pragma unroll
        for (int e = 0; e < 8; ++e) sf[e] = (__bf16)dp[8 * u + e];
        const int kb = kt * 32 + 16 * u;
#pragma unroll
        for (int dt = 0; dt < HS / 32; ++dt) {
          v4i16 rv[2];
#pragma unroll
          for (int t = 0; t < 2; ++t)
            rv[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(lbase + tr_off<RB>(toff[dt], t) + kb * RB));
          typedef short v8i16 __attribute__((ext_vector_type(8)));
          const v8i16 kv = {rv[0][0], rv[0][1], rv[0][2], rv[0][3],
                            rv[1][0], rv[1][1], rv[1][2], rv[1][3]};
          dq[dt] = mfma32(__builtin_bit_cast(bf16x8, kv), sf, dq[dt]);
        }
      }
    }
  };

  // keep bits: the word of tile it + 1 is loaded during tile it (before its
  // ring loads, so the next ring wait covers it)
  const KeepBitsLayout kl(T);
  uint32_t kw = 0;
  if constexpr (DROP) kw = keepq[kl.q_index(bh, 0, hi, myq)];
  auto next_keep = [&](int jn) -> uint32_t {
    if constexpr (DROP) {
      if (jn >= 0) return keepq[kl.q_index(bh, jn / BKV, hi, myq)];
    }
    return 0u;
  };
  const int n_full = min(nkv, (qt * 128) / BKV);
  int it = 0;
  for (; it < n_full; ++it) {
    wait_vmcnt<0>();
    bar_nofence();
    const int jn = it + 1 < nkv ? (it + 1) * BKV : -1;
    const uint32_t kn = next_keep(jn);
    tile(std::integral_constant<bool, false>{}, smem + (it & 1) * STAGE,
         smem + ((it + 1) & 1) * STAGE, jn, it * BKV, kw);
    kw = kn;
  }
  for (; it < nkv; ++it) {
    wait_vmcnt<0>();
    bar_nofence();
    const int jn = it + 1 < nkv ? (it + 1) * BKV : -1;
    const int j0 = it * BKV;
    char* wr = smem + ((it + 1) & 1) * STAGE;
    const uint32_t kn = next_keep(jn);
    if (j0 <= q0 + 31)
      tile(std::integral_constant<bool, true>{}, smem + (it & 1) * STAGE, wr, jn, j0, kw);
    else if (jn >= 0)
      issue(wr, jn);
    kw = kn;
  }

  if (myq < T) {
    bf16_t* row = dqkv + ((size_t)b * T + myq) * 3 * C + (size_t)h * HS;
#pragma unroll
    for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        uint2 w;
        w.x = pack_bf16x2(dq[dt][4 * g] * scale, dq[dt][4 * g + 1] * scale);
        w.y = pack_bf16x2(dq[dt][4 * g + 2] * scale, dq[dt][4 * g + 3] * scale);
        *reinterpret_cast<uint2*>(row + d0) = w;
      }
  }
}

// ------------------------------------------------------------- dK / dV
// One block = 4 waves = 128 keys of one (b, h); wave w owns 32 keys (lane =
// key) and keeps k and v of its key as MFMA B operands.  Per 64-query tile:
// S = Q K^T and dP = dO V^T (queries on the MFMA rows), P = exp2(S * scale *
// log2 e - L), dS = P (dP - D) (with DROP: P z for dV, dP z in dS, the keep
// factors z from the forward's keep bits, key-major layout of keep_bits.cuh),
// dV^T += dO^T P and dK^T += Q^T dS.  Stage: Q tile, dO tile, then the 64
// queries' L (log2 units) and D (fp32).
template <int HS, bool DROP>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv2_bf16_kernel(
    const bf16_t* __restrict__ Qg, const bf16_t* __restrict__ Kg,
    const bf16_t* __restrict__ Vg, const bf16_t* __restrict__ dOg,
    const float* __restrict__ Lpad, const float* __restrict__ Dpad, bf16_t* __restrict__ dqkv,
    int H, int T, int Tpad, float scale, float scale_log2, DropParams drop,
    const uint32_t* __restrict__ keepk) {
  static_assert(HS == 32 || HS == 64, "head size");
  constexpr int BQ = 64;
  constexpr int TILE = BQ * HS * 2;    // bytes of one Q or dO tile
  // Q tile, dO tile, L and D of the 64 queries (512 B), and with DROP the
  // keep words of the block's 128 keys for the tile (2 x 512 B)
  constexpr int STAGE = 2 * TILE + 512 + (DROP ? 1024 : 0);
  constexpr int RB = HS * 2;
  constexpr int CPR = HS / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int LPW = TILE / 1024 / 4;
  __shared__ __align__(1024) char smem[2 * STAGE];

  const int bh = blockIdx.x;
  const int kblk = (int)blockIdx.y;  // small key blocks see the most queries: first
  const int b = bh / H, h = bh - b * H;
  const int C = H * HS;
  const size_t head = (size_t)bh * T * HS;
  const bf16_t* Qh = Qg + head;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;
  const int kb0 = kblk * 128;
  const int kw0 = kb0 + wid * 32;
  const int mykey = kw0 + (lane & 31);

  bf16x8 kf[HS / 16], vf[HS / 16];
#pragma unroll
  for (int kk = 0; kk < HS / 16; ++kk) {
    if (mykey < T) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(Kg + head + (size_t)mykey * HS + 16 * kk + 8 * hi);
      vf[kk] = *reinterpret_cast<const bf16x8*>(Vg + head + (size_t)mykey * HS + 16 * kk + 8 * hi);
    } else {
      kf[kk] = bf16x8{};
      vf[kk] = bf16x8{};
    }
  }
  floatx16 dk[HS / 32], dv[HS / 32];
#pragma unroll
  for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  int qoff[HS / 16];
#pragma unroll
  for (int kk = 0; kk < HS / 16; ++kk) {
    const int row = lane & 31;
    qoff[kk] = row * RB + (((2 * kk + hi) ^ kv_swz<HS>(row)) << 4);
  }
  const int G = lane >> 4, s16 = lane & 15;
  const int r0 = 4 * (G >> 1) + (s16 >> 2);
  // t = 1 (rows r0 + 8) flips chunk bit 1 of the swizzle: offset bit 5.
  int toff[HS / 32];
#pragma unroll
  for (int dt = 0; dt < HS / 32; ++dt) {
    const int d = dt * 32 + 16 * (G & 1) + 4 * (s16 & 3);
    toff[dt] = r0 * RB + (((d >> 3) ^ kv_swz<HS>(r0)) << 4) + ((d >> 2) & 1) * 8;
  }

  const int nqt = (T - kb0 + BQ - 1) / BQ;  // query tiles i0 = kb0, kb0 + 64, ...
  const float* Lrow = Lpad + (size_t)bh * Tpad;
  const float* Drow = Dpad + (size_t)bh * Tpad;
  const KeepBitsLayout kl(T);

  // Loop-invariant per-lane byte offsets of each load's (row, chunk), loads
  // through buffer resources: Q's (b, h) slab, and dO's rows of (b, h) (row
  // stride C, the head's HS columns; the resource ends after row T - 1's
  // columns, so rows past T read zeros).  A query tile at i0 adds the
  // wave-uniform offset of i0 rows.
  const bf16_t* dOh = dOg + (size_t)b * T * C + h * HS;
  const __amdgpu_buffer_rsrc_t rq = slab_rsrc(Qh, (uint32_t)T * HS * 2);
  const __amdgpu_buffer_rsrc_t ro = slab_rsrc(dOh, ((uint32_t)(T - 1) * C + HS) * 2);
  uint32_t q_off[LPW], o_off[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int row = (wid * LPW + q) * RPI + lane / CPR;
    const int c8 = ((lane % CPR) ^ kv_swz<HS>(row)) * 8;
    q_off[q] = (uint32_t)(row * HS + c8) * 2;
    o_off[q] = (uint32_t)(row * C + c8) * 2;
  }
  auto issue = [&](char* dst, int i0) {
    const uint32_t sq = (uint32_t)i0 * HS * 2, so = (uint32_t)i0 * C * 2;
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      char* base = dst + (wid * LPW + q) * 1024;
      buffer_to_lds16(rq, base, q_off[q], sq);
      buffer_to_lds16(ro, base + TILE, o_off[q], so);
    }
    // L and D of the 64 queries (rows padded to Tpad, so always in bounds):
    // lanes 0..15 of wave 0 fetch L, lanes 16..31 D, 16 bytes each
    if (wid == 0 && lane < 32) {
      const float* src = lane < 16 ? Lrow + i0 + 4 * lane : Drow + i0 + 4 * (lane - 16);
      __builtin_amdgcn_load_to_lds((void*)src, GA_LDS(dst + 2 * TILE), 16, 0, 0);
    }
    // keep words k_index(bh, i0 / 64, hi, kb0 .. kb0 + 127) (keys padded to
    // 128, so always in bounds): lane l of wave 1 fetches 4 keys of hi = l / 32
    if constexpr (DROP) {
      if (wid == 1) {
        const uint32_t* src = keepk + kl.k_index(bh, i0 / BQ, lane >> 5, kb0 + 4 * (lane & 31));
        __builtin_amdgcn_load_to_lds((void*)src, GA_LDS(dst + 2 * TILE + 512), 16, 0, 0);
      }
    }
  };
  issue(smem, kb0);

  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) const bf16x8 lds_b128;
  typedef float f4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) const f4v lds_f4;

  // MASK: the tile reaches the keys' diagonal; RAGGED: it may hold queries
  // at or past T (rows whose Q and dO read zeros, and whose L and D pad
  // entries are never written), which are zeroed explicitly
  auto tile = [&](auto mask_tag, auto ragged_tag, const char* __restrict__ rd,
                  char* __restrict__ wr, int in, int i0) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    if (in >= 0) issue(wr, in);
    const lds_char* lbase = (const lds_char*)rd;
    floatx16 s[2], dp[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[qh][r] = 0.f;
        dp[qh][r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < HS / 16; ++kk) {
        const bf16x8 qa = *(lds_b128*)(lbase + qoff[kk] + qh * 32 * RB);
        const bf16x8 ga = *(lds_b128*)(lbase + TILE + qoff[kk] + qh * 32 * RB);
        s[qh] = mfma32(qa, kf[kk], s[qh]);
        dp[qh] = mfma32(ga, vf[kk], dp[qh]);
      }
    }
    // lane = key mykey; register r of qh <-> query i0 + qh*32 + 8(r/4) + 4hi + r%4
    // this lane's keep bits of the query tile (bit 16qh + 4g + e)
    uint32_t kw = 0;
    if constexpr (DROP)
      kw = *(const __attribute__((address_space(3))) uint32_t*)(
          lbase + 2 * TILE + 512 + (hi * 128 + (mykey - kb0)) * 4);
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = qh * 32 + 8 * g + 4 * hi;
        const f4v Lv = *(lds_f4*)(lbase + 2 * TILE + ql * 4);
        const f4v Dv = *(lds_f4*)(lbase + 2 * TILE + 256 + ql * 4);
        const float Ls[4] = {Lv[0], Lv[1], Lv[2], Lv[3]}, Ds[4] = {Dv[0], Dv[1], Dv[2], Dv[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const int q = i0 + ql + e;
          float p = __builtin_amdgcn_exp2f(fmaf(s[qh][r], scale_log2, -Ls[e]));
          float dpv = dp[qh][r];
          if constexpr (DROP) {
            const float z = ((kw >> (16 * qh + r)) & 1u) ? drop.scale : 0.f;
            s[qh][r] = p * z;
            dp[qh][r] = p * (dpv * z - Ds[e]);
          } else {
            s[qh][r] = p;
            dp[qh][r] = p * (dpv - Ds[e]);
          }
          const bool dead = (RAGGED && q >= T) || (MASK && mykey > q);
          if (dead) {
            s[qh][r] = 0.f;
            dp[qh][r] = 0.f;
          }
        }
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS; transposing reads in the query order
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 pf, sf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[e] = (__bf16)s[qh][8 * u + e];
          sf[e] = (__bf16)dp[qh][8 * u + e];
        }
        const int qb = qh * 32 + 16 * u;
#pragma unroll
        for (int dt = 0; dt < HS / 32; ++dt) {
          v4i16 ro[2], rq[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            ro[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(lbase + TILE + tr_off<RB>(toff[dt], t) +
                                                           qb * RB));
            rq[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(lbase + tr_off<RB>(toff[dt], t) + qb * RB));
          }
          typedef short v8i16 __attribute__((ext_vector_type(8)));
          const v8i16 ov = {ro[0][0], ro[0][1], ro[0][2], ro[0][3],
                            ro[1][0], ro[1][1], ro[1][2], ro[1][3]};
          const v8i16 qv = {rq[0][0], rq[0][1], rq[0][2], rq[0][3],
                            rq[1][0], rq[1][1], rq[1][2], rq[1][3]};
          dv[dt] = mfma32(__builtin_bit_cast(bf16x8, ov), pf, dv[dt]);
          dk[dt] = mfma32(__builtin_bit_cast(bf16x8, qv), sf, dk[dt]);
        }
      }
  };

  // the first two query tiles reach the block's keys' diagonal; a wave skips
  // a tile wholly before its keys
  const int n_mask = min(nqt, 2);
  int it = 0;
  for (; it < n_mask; ++it) {
    wait_vmcnt<0>();
    bar_nofence();
    const int i0 = kb0 + it * BQ;
    const int in = it + 1 < nqt ? i0 + BQ : -1;
    char* wr = smem + ((it + 1) & 1) * STAGE;
    if (i0 + BQ - 1 >= kw0)
      tile(std::true_type{}, std::true_type{}, smem + (it & 1) * STAGE, wr, in, i0);
    else if (in >= 0)
      issue(wr, in);
  }
  for (; it < nqt; ++it) {
    wait_vmcnt<0>();
    bar_nofence();
    const int i0 = kb0 + it * BQ;
    const int in = it + 1 < nqt ? i0 + BQ : -1;
    char* rd = smem + (it & 1) * STAGE;
    char* wr = smem + ((it + 1) & 1) * STAGE;
    // (with dropout the kernel keeps one body: a second copy of the loop
    // body pushes it past the register file)
    if constexpr (!DROP) {
      if (i0 + BQ <= T) {
        tile(std::false_type{}, std::false_type{}, rd, wr, in, i0);
        continue;
      }
    }
    tile(std::false_type{}, std::true_type{}, rd, wr, in, i0);
  }

  if (mykey < T) {
    bf16_t* row = dqkv + ((size_t)b * T + mykey) * 3 * C + (size_t)h * HS;
#pragma unroll
    for (int dt = 0; dt < HS / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        uint2 wk, wv;
        wk.x = pack_bf16x2(dk[dt][4 * g] * scale, dk[dt][4 * g + 1] * scale);
        wk.y = pack_bf16x2(dk[dt][4 * g + 2] * scale, dk[dt][4 * g + 3] * scale);
        wv.x = pack_bf16x2(dv[dt][4 * g], dv[dt][4 * g + 1]);
        wv.y = pack_bf16x2(dv[dt][4 * g + 2], dv[dt][4 * g + 3]);
        *reinterpret_cast<uint2*>(row + C + d0) = wk;
        *reinterpret_cast<uint2*>(row + 2 * C + d0) = wv;
      }
  }
}

}  // namespace gpt_attn
