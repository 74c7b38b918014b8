// gemm3.cuh -- bf16 MFMA GEMM whose operand loads and MFMAs run on
// different SIMDs.
//
// C[m][n] = sum_k A(m,k) B(k,n), fp32 accumulation, handed to a staged
// epilogue (bias, activation, rounding, 16-byte runs of a row; or, for
// epilogues that read memory per run, acc + bias in fp32; gemm2.cuh).
// Operand layouts and LDS swizzles as in gemm2.cuh.
//
// Why.  On gfx950 a global load (direct-to-LDS or into registers) issued by a
// wave on a SIMD that is busy with MFMAs takes about twice as long to go
// through, while LDS reads and writes do not mind the MFMAs; when every wave
// both loads and multiplies (gemm2_kernel), a k-tile's operand loads add
// their whole time to its MFMA time.  Here the 8 waves of a block split by
// SIMD: waves 0 and 4 (which share a SIMD) only issue the ring's
// direct-to-LDS loads, the other six only read fragments and run MFMAs.  The
// block loses a quarter of the CU's matrix rate and gains loads that overlap
// the other three SIMDs' MFMAs.
//
// Ring: NSTAGE stages of (BM + BN) x BK; at step kt the loader waves wait for
// their loads of tile kt, a barrier publishes it, the loaders issue tile
// kt + NSTAGE - 1 into the stage read at step kt - 1 and the MFMA waves
// multiply tile kt.  The six MFMA waves form a WGM x WGN grid over the block
// tile.  A row-contiguous operand tile may hold any multiple of 8 columns:
// its chunk swizzle XORs only the chunks below the last multiple of 16.
#pragma once

#include "common.cuh"
#include "gemm2.cuh"

namespace gpt_attn {

constexpr int kG3Loaders = 2;  // waves 0 and 4
constexpr int kG3Waves = 8;

// Chunk slot <-> source chunk of a row-contiguous tile with CPR 16-byte
// chunks per k-row (an involution).  A transposing fragment read takes 4
// consecutive k-rows at the same columns; LDS has 64 four-byte banks, so a
// k-row of CPR chunks starts 4 CPR banks after the previous one.  When that is
// a multiple of 64 (CPR % 16 == 0) the 4 rows would hit the same banks and
// XOR by 0, 4, 8 or 12 chunks (64-byte steps, inside the aligned group of 16)
// spreads them; when it is 16 or 48 banks (CPR % 16 == 4 or 12, e.g. 288
// columns) the rows already fall 16 banks apart and a swizzle would put two of
// them back together; in the remaining cases the XOR goes over the chunks
// below the last multiple of 16.
template <int CPR>
__device__ __forceinline__ int rc_swz(int chunk, int krow) {
  if constexpr (CPR % 16 == 4 || CPR % 16 == 12) {
    return chunk;
  } else {
    constexpr int kFull = CPR & ~15;
    return chunk < kFull ? (chunk ^ ((krow & 3) << 2)) : chunk;
  }
}

// Per-lane source offsets (elements, at k0 = 0) of the 1 KB loads that
// loader li issues for one operand tile: loads li, li + 2, li + 4, ...
template <int ROWS, int BK, bool KC>
struct G3Off {
  static constexpr int kLoads = ROWS * BK * 2 / 1024;
  static constexpr int kPerWave = kLoads / kG3Loaders;
  static_assert(kLoads % kG3Loaders == 0, "tile loads split evenly over the loaders");
  int off[kPerWave];
  __device__ __forceinline__ void init(int ld, int li, int lane) {
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      const int inst = li + kG3Loaders * q;
      if (KC) {
        constexpr int CPK = BK / 8;
        const int row = inst * (64 / CPK) + lane / CPK;
        off[q] = row * ld + ((lane % CPK) ^ kc_swz<BK>(row)) * 8;
      } else {
        constexpr int CPR = ROWS / 8;
        const int idx = inst * 64 + lane;
        const int krow = idx / CPR;
        off[q] = krow * ld + rc_swz<CPR>(idx % CPR, krow) * 8;
      }
    }
  }
};

// Loader li's loads of one operand tile (ROWS x BK at row0, k0) into lds.
template <int ROWS, int BK, bool KC>
__device__ __forceinline__ void g3_issue(const bf16_t* __restrict__ src, int ld, int row0,
                                         int nrows, int k0, int kend, char* lds, int li,
                                         int lane, const G3Off<ROWS, BK, KC>& po) {
  constexpr int kPerWave = G3Off<ROWS, BK, KC>::kPerWave;
  if (row0 + ROWS <= nrows && k0 + BK <= kend) {
    const bf16_t* base = KC ? src + (size_t)row0 * ld + k0 : src + (size_t)k0 * ld + row0;
#pragma unroll
    for (int q = 0; q < kPerWave; ++q)
      __builtin_amdgcn_load_to_lds((void*)(base + po.off[q]),
                                   GA_LDS(lds + (li + kG3Loaders * q) * 1024), 16, 0, 0);
    return;
  }
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) {
    const int inst = li + kG3Loaders * q;
    const bf16_t* g;
    if (KC) {
      constexpr int CPK = BK / 8;
      const int row = inst * (64 / CPK) + lane / CPK;
      const int chunk = (lane % CPK) ^ kc_swz<BK>(row);
      const int gr = row0 + row, gk = k0 + chunk * 8;
      g = (gr < nrows && gk < kend) ? src + (size_t)gr * ld + gk
                                    : reinterpret_cast<const bf16_t*>(&g_zero16);
    } else {
      constexpr int CPR = ROWS / 8;
      const int idx = inst * 64 + lane;
      const int krow = idx / CPR;
      const int chunk = rc_swz<CPR>(idx % CPR, krow);
      const int gk = k0 + krow, gr = row0 + chunk * 8;
      g = (gk < kend && gr < nrows) ? src + (size_t)gk * ld + gr
                                    : reinterpret_cast<const bf16_t*>(&g_zero16);
    }
    __builtin_amdgcn_load_to_lds((void*)g, GA_LDS(lds + inst * 1024), 16, 0, 0);
  }
}

// MFMA operand fragment of rows rb..rb+31, k = 16 kk + 8 (lane / 32) + 0..7
// (gemm2's g2_frag with the row-contiguous swizzle above).
template <int ROWS, int BK, bool KC>
__device__ __forceinline__ bf16x8 g3_frag(const char* lds, int rb, int kk, int lane) {
  if constexpr (KC) {
    return g2_frag<ROWS, BK, true>(lds, rb, kk, lane);
  } else {
    constexpr int CPR = ROWS / 8;
    const int G = lane >> 4, s = lane & 15;
    const int h = G >> 1, nsub = G & 1;
    const int n = rb + 16 * nsub + 4 * (s & 3);
    const int chunk = n >> 3, half = (n >> 2) & 1;
    v4i16 r[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int krow = 16 * kk + 8 * h + 4 * t + (s >> 2);
      const char* p = lds + krow * (ROWS * 2) + (rc_swz<CPR>(chunk, krow) << 4) + half * 8;
      r[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GA_LDS4(p));
    }
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    v8i16 c = {r[0][0], r[0][1], r[0][2], r[0][3], r[1][0], r[1][1], r[1][2], r[1][3]};
    return __builtin_bit_cast(bf16x8, c);
  }
}

// fp32-staged epilogue block (epilogues that read memory per run, e.g. a
// residual): the LDS block cf [32][BN + 4] holds acc + bias of tile rows
// 32 i .. 32 i + 31; all eight waves hand its 8-column runs to store8f, with
// the epilogue's Extra8 of all their runs loaded before the first store (a
// load after a store waits for it: they may alias).
template <int BN, class Epi>
__device__ __forceinline__ void g3_store_f32_block(const float* cf, const Epi& epi, int i, int m0,
                                                   int n0, int M, int N, int tid) {
  constexpr int SPF = BN + 4;
  constexpr int kRuns = 32 * BN / 8;
  constexpr int kPass = (kRuns + 64 * kG3Waves - 1) / (64 * kG3Waves);
  typename Epi::Extra8 ex[kPass];
#pragma unroll
  for (int p = 0; p < kPass; ++p) {
    const int c = tid + p * 64 * kG3Waves;
    const int m = m0 + i * 32 + c / (BN / 8), n = n0 + (c % (BN / 8)) * 8;
    ex[p] = epi.extra8(m, n, c < kRuns && m < M && n < N);
  }
#pragma unroll
  for (int p = 0; p < kPass; ++p) {
    const int c = tid + p * 64 * kG3Waves;
    const int rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
    const int m = m0 + i * 32 + rl, n = n0 + cl;
    if (c < kRuns && m < M && n < N) {
      const float4 a = *reinterpret_cast<const float4*>(cf + rl * SPF + cl);
      const float4 b = *reinterpret_cast<const float4*>(cf + rl * SPF + cl + 4);
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      epi.store8f(m, n, v, ex[p]);
    }
  }
}

template <int BM, int BN, int BK, int NSTAGE, bool A_KC, bool B_KC, int WGM, int WGN, class Epi>
__global__ __launch_bounds__(64 * kG3Waves) void gemm3_kernel(const bf16_t* __restrict__ A,
                                                              int lda,
                                                              const bf16_t* __restrict__ Bm,
                                                              int ldb, int M, int N, int K,
                                                              Epi epi) {
  static_assert(WGM * WGN == kG3Waves - kG3Loaders, "six MFMA waves");
  static_assert(Staged<Epi>::value, "staged epilogues");
  constexpr bool kF32 = StagedF32<Epi>::value;
  static_assert(!(kF32 && Store8All<Epi>::value), "store8_all goes with the bf16 staging");
  static_assert(!kF32 || WGM == 1, "fp32 staging goes by 32-row blocks of a one-row wave grid");
  static_assert(BK == 64 || BK == 32, "BK");
  static_assert(B_KC || (BN / 8) % 2 == 0, "row-contiguous tile");
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  constexpr int kA = BM * BK * 2, kB = BN * BK * 2;
  constexpr int kStage = kA + kB;
  constexpr int kRing = NSTAGE * kStage;
  constexpr int SP = BN + 8;  // staged epilogue pitch (elements)
  constexpr int kEpiBytes = BM * SP * 2;
  constexpr int SPF = BN + 4;  // fp32 staging pitch (floats), 32 rows at a time
  static_assert(kF32 ? 32 * SPF * 4 <= kRing : kEpiBytes <= kRing,
                "the staged tile reuses the ring");
  constexpr int kBiasOff = (kRing + 15) / 16 * 16;
  static_assert(kBiasOff + BN * 2 <= 160 * 1024, "LDS");
  constexpr int kLoadsA = G3Off<BM, BK, A_KC>::kPerWave, kLoadsB = G3Off<BN, BK, B_KC>::kPerWave;
  constexpr int kLoads = kLoadsA + kLoadsB;  // per loader wave per stage
  static_assert(kLoads * (NSTAGE - 1) < 64, "vmcnt range");
  __shared__ __align__(1024) char smem[kBiasOff + BN * 2];

  const int tiles_n = (N + BN - 1) / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  // each XCD's run of tiles covers a band of row tiles, column-major inside
  // the band (gemm2_kernel)
  const int tiles_m = (M + BM - 1) / BM;
  const int band = max(1, tiles_m / 8);
  const int bi = tile / (band * tiles_n), loc = tile - bi * band * tiles_n;
  const int rows = min(band, tiles_m - bi * band);
  const int m0 = (bi * band + loc % rows) * BM, n0 = (loc / rows) * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = (wid & 3) == 0;
  const int li = wid >> 2;                               // loader index
  const int ci = wid - 1 - (wid > 4 ? 1 : 0);            // MFMA wave index 0..5
  const int wm = ci / WGN, wn = ci % WGN;
  const int nk = (K + BK - 1) / BK;

  bf16_t* ct = reinterpret_cast<bf16_t*>(smem);
  float* cf = reinterpret_cast<float*>(smem);
  // The two roles run separate loops with the same barriers, so that the
  // loaders' offsets and the accumulators are never live together.
  if (loader) {
    G3Off<BM, BK, A_KC> pa;
    G3Off<BN, BK, B_KC> pb;
    // bias columns n0 .. n0+BN-1 straight to LDS, before the ring loads, so
    // the ring's waits cover it (lanes past the bias read the zero block)
    static_assert(BN % 8 == 0 && BN / 8 <= 64, "bias tile");
    if (li == 0 && lane < BN / 8) {
      const bf16_t* bp = epi.bias_ptr();
      const int n = n0 + 8 * lane;
      const bf16_t* g = (bp && n < N) ? bp + n : reinterpret_cast<const bf16_t*>(&g_zero16);
      __builtin_amdgcn_load_to_lds((void*)g, GA_LDS(smem + kBiasOff), 16, 0, 0);
    }
    pa.init(lda, li, lane);
    pb.init(ldb, li, lane);
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < nk) {
        char* sa = smem + s * kStage;
        g3_issue<BM, BK, A_KC>(A, lda, m0, M, s * BK, K, sa, li, lane, pa);
        g3_issue<BN, BK, B_KC>(Bm, ldb, n0, N, s * BK, K, sa + kA, li, lane, pb);
      }
    for (int kt = 0; kt < nk; ++kt) {
      // tile kt is complete once at most (later tiles issued) x loads remain
      const int later = min(nk - 1, kt + NSTAGE - 2) - kt;
      if (later >= NSTAGE - 2) wait_vmcnt<kLoads * (NSTAGE - 2)>();
      else if (NSTAGE > 3 && later == 2) wait_vmcnt<kLoads * 2>();
      else if (later == 1) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
      bar_nofence();
      const int kn = kt + NSTAGE - 1;
      if (kn < nk) {
        char* sw = smem + (kn % NSTAGE) * kStage;
        g3_issue<BM, BK, A_KC>(A, lda, m0, M, kn * BK, K, sw, li, lane, pa);
        g3_issue<BN, BK, B_KC>(Bm, ldb, n0, N, kn * BK, K, sw + kA, li, lane, pb);
      }
    }
    if constexpr (kF32) {
#pragma unroll 1
      for (int i = 0; i < MT; ++i) {
        bar_nofence();  // the ring / the previous block's runs are free
        bar_after_lds_writes();
        g3_store_f32_block<BN>(cf, epi, i, m0, n0, M, N, tid);
      }
      return;
    }
    bar_nofence();  // the ring is free for the staged tile
  } else {
    floatx16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      bar_nofence();
      const char* rd = smem + (kt % NSTAGE) * kStage;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 af[MT], bfr[NT];
#pragma unroll
        for (int i = 0; i < MT; ++i) af[i] = g3_frag<BM, BK, A_KC>(rd, wm * WTM + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < NT; ++j)
          bfr[j] = g3_frag<BN, BK, B_KC>(rd + kA, wn * WTN + j * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
      }
    }
    if constexpr (kF32) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        bar_nofence();  // the ring / the previous block's runs are free
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int cl = wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
            const uint2 bu = *reinterpret_cast<const uint2*>(smem + kBiasOff + cl * 2);
            const float b[4] = {bf2f(bu.x & 0xffff), bf2f(bu.x >> 16), bf2f(bu.y & 0xffff),
                                bf2f(bu.y >> 16)};
            *reinterpret_cast<float4*>(cf + (lane & 31) * SPF + cl) =
                make_float4(acc[i][j][4 * g] + b[0], acc[i][j][4 * g + 1] + b[1],
                            acc[i][j][4 * g + 2] + b[2], acc[i][j][4 * g + 3] + b[3]);
          }
        bar_after_lds_writes();
        g3_store_f32_block<BN>(cf, epi, i, m0, n0, M, N, tid);
      }
      return;
    }
    bar_nofence();  // every wave is done with the ring
    // staged epilogue: bias + acc (rounded, with the epilogue's activation)
    // into an LDS tile [BM][BN + 8] over the ring
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cl = wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
        const uint2 bu = *reinterpret_cast<const uint2*>(smem + kBiasOff + cl * 2);
        const float b[4] = {bf2f(bu.x & 0xffff), bf2f(bu.x >> 16), bf2f(bu.y & 0xffff),
                            bf2f(bu.y >> 16)};
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const int rl = wm * WTM + i * 32 + (lane & 31);
          constexpr int ACT = ActOf<Epi>::value;
          uint2 w;
          w.x = pack_bf16x2(apply_act<ACT>(acc[i][j][4 * g] + b[0]),
                            apply_act<ACT>(acc[i][j][4 * g + 1] + b[1]));
          w.y = pack_bf16x2(apply_act<ACT>(acc[i][j][4 * g + 2] + b[2]),
                            apply_act<ACT>(acc[i][j][4 * g + 3] + b[3]));
          *reinterpret_cast<uint2*>(ct + rl * SP + cl) = w;
        }
      }
  }
  // all eight waves store 16-byte runs of the staged rows
  if constexpr (!kF32) {
    bar_after_lds_writes();
    constexpr int kChunks = BM * BN / 8;
    if constexpr (Store8All<Epi>::value) {
      // every lane in every pass (the epilogue combines lanes); the
      // epilogue's own operands of all passes are loaded before the first
      // store, which later loads would wait behind (they may alias)
      static_assert(kChunks % (64 * kG3Waves) == 0, "store8_all needs every lane in every pass");
      constexpr int kPass = kChunks / (64 * kG3Waves);
      typename Epi::Extra ex[kPass];
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        const int c = tid + p * 64 * kG3Waves;
        const int m = m0 + c / (BN / 8), n = n0 + (c % (BN / 8)) * 8;
        ex[p] = epi.extra(m, n, m < M && n < N);
      }
#pragma unroll
      for (int p = 0; p < kPass; ++p) {
        const int c = tid + p * 64 * kG3Waves;
        const int rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
        const int m = m0 + rl, n = n0 + cl;
        epi.store8_all(m, n, *reinterpret_cast<const uint4*>(ct + rl * SP + cl),
                       m < M && n < N, lane, ex[p]);
      }
    } else {
      for (int c = tid; c < kChunks; c += 64 * kG3Waves) {
        const int rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
        const int m = m0 + rl, n = n0 + cl;
        if (m < M && n < N) epi.store8(m, n, *reinterpret_cast<const uint4*>(ct + rl * SP + cl));
      }
    }
  }
}

// Launch over all output tiles (no split of K).  Requires N % 8 == 0, K % 8
// == 0 for a k-contiguous operand and the row count % 8 == 0 for a
// row-contiguous one (as gemm2).
template <int BM, int BN, int NSTAGE, int BK, int WGM, int WGN, bool A_KC, bool B_KC, class Epi>
inline void launch_gemm3(const bf16_t* A, int lda, const bf16_t* B, int ldb, int M, int N, int K,
                         const Epi& epi, hipStream_t st) {
  const int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (grid == 0 || K <= 0) return;
  hipLaunchKernelGGL((gemm3_kernel<BM, BN, BK, NSTAGE, A_KC, B_KC, WGM, WGN, Epi>), dim3(grid),
                     dim3(64 * kG3Waves), 0, st, A, lda, B, ldb, M, N, K, epi);
}

}  // namespace gpt_attn
