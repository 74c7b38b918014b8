// gemm2.cuh -- pipelined bf16 MFMA GEMM for gfx950.
//
// C[m][n] = sum_k A(m,k) B(k,n) with fp32 accumulation, handed to an epilogue
// in runs of 4 consecutive columns.  Operand layouts (template flags):
//   A_KC: A(m,k) = A[m*lda + k]  (k contiguous)   else A(m,k) = A[k*lda + m]
//   B_KC: B(k,n) = B[n*ldb + k]  (k contiguous)   else B(k,n) = B[k*ldb + n]
//
// Data movement.  Operand tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (no register staging), into an NSTAGE-deep ring:
// the loads for k-tile kt+NSTAGE-1 are in flight while tile kt is multiplied.
// Each wave waits only for its own oldest loads (s_waitcnt vmcnt(n)) and a
// bare s_barrier publishes the tile; no fence drains the ring.
//
// LDS layouts (16-byte chunks, XOR-swizzled so MFMA operand reads spread over
// the banks):
//   k-contiguous operand: [row][BK], chunk c of row r at slot c ^ kc_swz(r);
//     an MFMA fragment (32 rows x 16 k) is one ds_read_b128 per lane.
//   row-contiguous operand: [BK][ROWS], chunk c of k-row r at slot
//     c ^ 4*(r & 3); a fragment is two ds_read_b64_tr_b16 per lane.  Within a
//     group of 16 lanes that instruction hands output lane j element e =
//     the (j%4)-th 16-bit value fetched by source lane 4e + j/4; so source lane
//     s pointing at row kb + s/4, column nb + 4(s%4) delivers to lane j the
//     four k values kb..kb+3 of column nb + j -- the MFMA operand layout.
//
// MFMA.  v_mfma_f32_32x32x16_bf16 with the operands swapped (B fragment as
// the "A" input), so each accumulator tile is D^T: lane l holds row
// m = l%32 and, in register group g, the four consecutive columns
// 8g + 4(l/32) + 0..3 -- stored directly as 8 (bf16) or 16 (fp32) bytes.
//
// WGM x WGN waves (64 threads each); block tile BM x BN; split-K over
// grid.y.  Chunks outside the matrix (ragged M, N or K) read a 16-byte zero
// block.  Requires N % 8 == 0, K % 8 == 0 for a k-contiguous operand and the
// row count % 8 == 0 for a row-contiguous one.
#pragma once

#include "common.cuh"
#include "gemm.cuh"

namespace gpt_attn {

__device__ __align__(16) static const uint4 g_zero16 = {0u, 0u, 0u, 0u};

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define GA_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define GA_LDS4(p) ((__attribute__((address_space(3))) v4i16*)(p))

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_barrier without a memory fence (the ring is published by the waits
// above), fenced against compiler reordering of LDS accesses.
__device__ __forceinline__ void bar_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_barrier after this wave's LDS writes have completed (lgkmcnt 0): the
// barrier alone does not order one wave's ds_write before another wave's
// ds_read of the same address.
__device__ __forceinline__ void bar_after_lds_writes() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int BN, int BK, int NSTAGE, bool A_KC, bool B_KC, int NW = 4>
struct Gemm2Cfg {
  static_assert(BK == 64 || BK == 32, "BK");
  static constexpr int kA = BM * BK * 2;            // bytes of one A stage
  static constexpr int kB = BN * BK * 2;            // bytes of one B stage
  static constexpr int kStage = kA + kB;
  static constexpr int kSmem = NSTAGE * kStage;
  static constexpr int kLoadsA = kA / 1024 / NW;    // 1 KB loads per wave
  static constexpr int kLoadsB = kB / 1024 / NW;
  static constexpr int kLoads = kLoadsA + kLoadsB;  // per wave per stage
  static_assert(kA % (1024 * NW) == 0 && kB % (1024 * NW) == 0, "tile too small");
  static_assert(kLoads * (NSTAGE - 1) < 64, "vmcnt range");
  static_assert(kSmem <= 160 * 1024, "LDS");
};

// Issue the global->LDS loads of one operand tile (ROWS x BK) for this wave.
// KC: source (row, k) at src[row*ld + k]; RC: at src[k*ld + row].
// Slot swizzle of a k-contiguous tile: chunk c of row r lives at c ^ kc_swz(r).
// LDS has 64 four-byte banks (256-byte bank lines); a fragment read serves
// 16 lanes = 16 consecutive rows at one chunk per pass.  BK = 64 (128-byte
// rows, two per bank line): rows of equal parity need distinct slots, so
// the swizzle is (r >> 1) & 7.  BK = 32 (64-byte rows, four per line):
// (r >> 2) & 3.
template <int BK>
__device__ __forceinline__ int kc_swz(int row) {
  return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

// A row-contiguous tile's k-rows hold ROWS/8 chunks; the swizzle XORs the
// chunk index with 0, 4, 8 or 12, which maps [0, ROWS/8) onto itself when
// ROWS/8 is a multiple of 16.
template <int ROWS, int BK, bool KC>
__device__ __forceinline__ void g2_issue_check() {
  static_assert(KC || (ROWS % 128 == 0), "row-contiguous operand tiles need 128 | ROWS");
}

// Per-lane source offsets of one operand tile's loads (element offsets at
// k0 = 0 relative to the tile's first row / column); loop-invariant, so a
// k-tile adds only its k offset.
template <int ROWS, int BK, bool KC, int NW = 4>
struct G2Off {
  static constexpr int kPerWave = ROWS * BK * 2 / 1024 / NW;
  int off[kPerWave];
  __device__ __forceinline__ void init(int ld, int wid, int lane) {
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      const int inst = wid * kPerWave + q;
      if (KC) {
        constexpr int CPK = BK / 8;
        const int row = inst * (64 / CPK) + lane / CPK;
        off[q] = row * ld + ((lane % CPK) ^ kc_swz<BK>(row)) * 8;
      } else {
        constexpr int CPR = ROWS / 8;
        const int idx = inst * 64 + lane;  // chunk index within the tile
        const int krow = idx / CPR;
        off[q] = krow * ld + ((idx % CPR) ^ ((krow & 3) << 2)) * 8;
      }
    }
  }
};

// Issue the global->LDS loads of one operand tile (ROWS x BK) for this wave.
// KC: source (row, k) at src[row*ld + k]; RC: at src[k*ld + row].  A tile
// wholly inside the matrix (rows and k) takes the precomputed offsets; a
// ragged one checks every chunk and reads the zero block outside.
template <int ROWS, int BK, bool KC, int NW = 4>
__device__ __forceinline__ void g2_issue(const bf16_t* __restrict__ src, int ld, int row0,
                                         int nrows, int k0, int kend, char* lds, int wid,
                                         int lane, const G2Off<ROWS, BK, KC, NW>& po) {
  constexpr int kPerWave = ROWS * BK * 2 / 1024 / NW;
  g2_issue_check<ROWS, BK, KC>();
  if (row0 + ROWS <= nrows && k0 + BK <= kend) {
    const bf16_t* base = KC ? src + (size_t)row0 * ld + k0 : src + (size_t)k0 * ld + row0;
#pragma unroll
    for (int q = 0; q < kPerWave; ++q)
      __builtin_amdgcn_load_to_lds((void*)(base + po.off[q]),
                                   GA_LDS(lds + (wid * kPerWave + q) * 1024), 16, 0, 0);
    return;
  }
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) {
    const int inst = wid * kPerWave + q;  // 1 KB block index within the tile
    const bf16_t* g;
    if (KC) {
      // 1024 / (2 BK) rows of BK k per instruction; lane -> (row, slot)
      constexpr int CPK = BK / 8;  // chunks per row
      const int row = inst * (64 / CPK) + lane / CPK;
      const int slot = lane % CPK;
      const int chunk = slot ^ kc_swz<BK>(row);
      const int gr = row0 + row, gk = k0 + chunk * 8;
      g = (gr < nrows && gk < kend) ? src + (size_t)gr * ld + gk
                                    : reinterpret_cast<const bf16_t*>(&g_zero16);
    } else {
      constexpr int CPR = ROWS / 8;               // chunks per k-row
      const int idx = inst * 64 + lane;           // chunk index within the tile
      const int krow = idx / CPR;
      const int slot = idx % CPR;
      const int chunk = slot ^ ((krow & 3) << 2);
      const int gk = k0 + krow, gr = row0 + chunk * 8;
      g = (gk < kend && gr < nrows) ? src + (size_t)gk * ld + gr
                                    : reinterpret_cast<const bf16_t*>(&g_zero16);
    }
    __builtin_amdgcn_load_to_lds((void*)g, GA_LDS(lds + inst * 1024), 16, 0, 0);
  }
}

// MFMA operand fragment: rows rb..rb+31 of the tile, k = 16*kk + 8*(lane/32) + 0..7.
// (kc_swz, the k-contiguous swizzle, is defined above g2_issue.)
template <int ROWS, int BK, bool KC>
__device__ __forceinline__ bf16x8 g2_frag(const char* lds, int rb, int kk, int lane) {
  if (KC) {
    const int row = rb + (lane & 31);
    const int chunk = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(lds + row * (BK * 2) + ((chunk ^ kc_swz<BK>(row)) << 4));
  } else {
    const int G = lane >> 4, s = lane & 15;
    const int h = G >> 1, nsub = G & 1;
    const int n = rb + 16 * nsub + 4 * (s & 3);
    const int chunk = n >> 3, half = (n >> 2) & 1;
    v4i16 r[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int krow = 16 * kk + 8 * h + 4 * t + (s >> 2);
      const char* p = lds + krow * (ROWS * 2) + ((chunk ^ ((krow & 3) << 2)) << 4) + half * 8;
      r[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(GA_LDS4(p));
    }
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    v8i16 c = {r[0][0], r[0][1], r[0][2], r[0][3], r[1][0], r[1][1], r[1][2], r[1][3]};
    return __builtin_bit_cast(bf16x8, c);
  }
}

// Epilogues receive (m, n, v[4]) for columns n..n+3 (n % 4 == 0).
struct Epi2RowMajor {
  bf16_t* out;
  int ldc;
  const bf16_t* bias;  // may be NULL
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      const uint2 u = *reinterpret_cast<const uint2*>(bias + n);
      b[0] = bf2f(u.x & 0xffff); b[1] = bf2f(u.x >> 16);
      b[2] = bf2f(u.y & 0xffff); b[3] = bf2f(u.y >> 16);
    }
    uint2 w;
    w.x = pack_bf16x2(v[0] + b[0], v[1] + b[1]);
    w.y = pack_bf16x2(v[2] + b[2], v[3] + b[3]);
    *reinterpret_cast<uint2*>(out + (size_t)m * ldc + n) = w;
  }
  // staged path: bias is added before rounding into the LDS tile; the
  // output (y, dx) is a final one, stored non-temporally
  static constexpr bool kStaged = true;
  __device__ __forceinline__ const bf16_t* bias_ptr() const { return bias; }
  __device__ __forceinline__ void store8(int m, int n, uint4 w) const {
    store16_stream(out + (size_t)m * ldc + n, w);
  }
};

// c_attn epilogue: bias, rounding, and the scatter of column n of row
// m = b*T + t to qkv[s][b][h][t][d] (s = n / C, h = (n % C) / hs, d = n % hs).
// The kernel asks for row and column offsets once per 32-row / 32-column
// block (hs is a multiple of 32, so a 32-column block lies in one head) and
// adds the per-lane remainder.
struct Epi2QKV {
  bf16_t* qkv;
  const bf16_t* bias;  // [3C] or NULL
  int B, T, C, H, hs;
  int wt;  // staged stores written through L2 (the tensor spans < 2^31 bytes)
  static constexpr bool kSplitOffsets = true;
  __device__ __forceinline__ size_t row_off(int m) const {  // (b, t) part
    const int bb = m / T, t = m - bb * T;
    return ((size_t)bb * H * T + t) * hs;
  }
  __device__ __forceinline__ size_t col_off(int n) const {  // (s, h, d) part
    const int s = n / C, rem = n - s * C;
    const int h = rem / hs, d = rem - h * hs;
    return (size_t)s * B * H * T * hs + (size_t)h * T * hs + d;
  }
  __device__ __forceinline__ void store(size_t off, int n, const float* v) const {
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      const uint2 u = *reinterpret_cast<const uint2*>(bias + n);
      b[0] = bf2f(u.x & 0xffff); b[1] = bf2f(u.x >> 16);
      b[2] = bf2f(u.y & 0xffff); b[3] = bf2f(u.y >> 16);
    }
    uint2 w;
    w.x = pack_bf16x2(v[0] + b[0], v[1] + b[1]);
    w.y = pack_bf16x2(v[2] + b[2], v[3] + b[3]);
    *reinterpret_cast<uint2*>(qkv + off) = w;
  }
  static constexpr bool kStaged = true;
  __device__ __forceinline__ const bf16_t* bias_ptr() const { return bias; }
  __device__ __forceinline__ void store8(int m, int n, uint4 w) const {
    const size_t off = row_off(m) + col_off(n);
    if (wt)
      store16_wt(qkv, (uint32_t)(off * 2), w);
    else
      *reinterpret_cast<uint4*>(qkv + off) = w;
  }
};

// Exact GELU, g(v) = v * Phi(v) = v/2 * (1 + erf(v / sqrt(2))) (page "nanoGPT
// architecture explained step by step", section 4), with erf from Abramowitz
// and Stegun, Handbook of Mathematical Functions, formula 7.1.26: for a >= 0,
// erfc(a) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-a^2) + e(a),
// t = 1 / (1 + p a), |e(a)| <= 1.5e-7.  With a = |v| / sqrt(2),
// g(v) = v - v/2 erfc(a) for v >= 0 and v/2 erfc(a) for v < 0, so the negative
// tail is a product (no cancellation in 1 + erf); |g - exact| <= |v| 7.5e-8
// before rounding, far below the bf16 step of the stored activation.  Both
// signs in one form: g(v) = max(v, 0) - |v|/2 erfc(a).  The constants absorb
// the scalings: with s = sqrt(log2 e) and a' = s a, exp(-a^2) = 2^(-a'^2),
// t = 1 / (1 + (p / s) a'), and the five coefficients carry the 1/2, so a
// value costs 13 VALU operations besides its rcp and exp2.
__device__ __forceinline__ float gelu_erf(float v) {
  constexpr double kS = 1.2011224087864498;  // sqrt(log2 e)
  const float ap = fabsf(v) * (float)(0.70710678118654752 * kS);
  const float t = __builtin_amdgcn_rcpf(fmaf((float)(0.3275911 / kS), ap, 1.f));
  float q = fmaf((float)(0.5 * 1.061405429), t, (float)(0.5 * -1.453152027));
  q = fmaf(q, t, (float)(0.5 * 1.421413741));
  q = fmaf(q, t, (float)(0.5 * -0.284496736));
  q = fmaf(q, t, (float)(0.5 * 0.254829592));
  const float half_erfc = q * t * __builtin_amdgcn_exp2f(-(ap * ap));
  return fmaf(-fabsf(v), half_erfc, fmaxf(v, 0.f));
}

// MLP c_fc epilogue: bias, exact GELU, rounding; row-major [M][ldc].
struct Epi2Gelu {
  bf16_t* out;
  int ldc;
  const bf16_t* bias;  // may be NULL
  static constexpr int kAct = 1;
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
      const uint2 u = *reinterpret_cast<const uint2*>(bias + n);
      b[0] = bf2f(u.x & 0xffff); b[1] = bf2f(u.x >> 16);
      b[2] = bf2f(u.y & 0xffff); b[3] = bf2f(u.y >> 16);
    }
    uint2 w;
    w.x = pack_bf16x2(gelu_erf(v[0] + b[0]), gelu_erf(v[1] + b[1]));
    w.y = pack_bf16x2(gelu_erf(v[2] + b[2]), gelu_erf(v[3] + b[3]));
    *reinterpret_cast<uint2*>(out + (size_t)m * ldc + n) = w;
  }
  static constexpr bool kStaged = true;
  __device__ __forceinline__ const bf16_t* bias_ptr() const { return bias; }
  __device__ __forceinline__ void store8(int m, int n, uint4 w) const {
    *reinterpret_cast<uint4*>(out + (size_t)m * ldc + n) = w;
  }
};

// Activation applied after the bias in the staged epilogue (0: none).
template <class Epi, class = void>
struct ActOf { static constexpr int value = 0; };
template <class Epi>
struct ActOf<Epi, decltype(void(Epi::kAct))> { static constexpr int value = Epi::kAct; };
template <int ACT>
__device__ __forceinline__ float apply_act(float v) { return ACT == 1 ? gelu_erf(v) : v; }

template <class Epi, class = void>
struct Staged { static constexpr bool value = false; };
template <class Epi>
struct Staged<Epi, decltype(void(Epi::kStaged))> { static constexpr bool value = Epi::kStaged; };

// kStore8All: the staged epilogue calls store8_all(m, n, w, in_range, lane,
// extra) from every lane of every wave (with in_range false outside the
// matrix), so the epilogue may combine values across lanes; `extra` is what
// the epilogue's extra(m, n, in_range) loaded for that chunk beforehand.
template <class Epi, class = void>
struct Store8All { static constexpr bool value = false; };
template <class Epi>
struct Store8All<Epi, decltype(void(Epi::kStore8All))> {
  static constexpr bool value = Epi::kStore8All;
};

// kStagedF32: the staged epilogue keeps acc + bias in fp32 (one half of the
// tile's rows at a time, so the fp32 half-tile fits the ring's LDS) and hands
// each 8-column run to store8f(m, n, v[8], extra) to round once.  Such an
// epilogue reads memory per run (a residual): it declares Epi::Extra8 and
// extra8(m, n, in_range), and the runs of all passes are loaded before the
// first store, since a load issued between stores waits for them (they may
// alias, and stores count in vmcnt).
template <class Epi, class = void>
struct StagedF32 { static constexpr bool value = false; };
template <class Epi>
struct StagedF32<Epi, decltype(void(Epi::kStagedF32))> {
  static constexpr bool value = Epi::kStagedF32;
};

template <class Epi, class = void>
struct SplitOffsets { static constexpr bool value = false; };
template <class Epi>
struct SplitOffsets<Epi, decltype(void(Epi::kSplitOffsets))> {
  static constexpr bool value = Epi::kSplitOffsets;
};

struct Epi2Partial {
  float* part;
  int ldc;
  size_t split_stride;
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    *reinterpret_cast<float4*>(part + (size_t)blockIdx.y * split_stride + (size_t)m * ldc + n) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Split-K partials that also carry the column sums of B over the slice's
// k-range (a weight gradient's bias gradient: B is the output gradient, and
// db[n] = sum_k B(k, n)).  With `colsum` set, the blocks of the first row
// tile add up the B fragments their first wave row reads for the MFMAs and
// write the sums to row M of the slice's partial block (split_stride covers
// M + 1 rows).
struct Epi2PartialCS {
  float* part;
  int ldc;
  size_t split_stride;
  int M;
  int colsum;
  static constexpr bool kColSumB = true;
  __device__ __forceinline__ void operator()(int m, int n, const float* v) const {
    *reinterpret_cast<float4*>(part + (size_t)blockIdx.y * split_stride + (size_t)m * ldc + n) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ void store_colsum(int n, float v) const {
    part[(size_t)blockIdx.y * split_stride + (size_t)M * ldc + n] = v;
  }
};

template <class Epi, class = void>
struct ColSumB { static constexpr bool value = false; };
template <class Epi>
struct ColSumB<Epi, decltype(void(Epi::kColSumB))> { static constexpr bool value = Epi::kColSumB; };

// Sum of the 8 bf16 values of an MFMA operand fragment, in fp32.
__device__ __forceinline__ float frag_sum8(const bf16x8& f) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += (float)f[e];
  return s;
}

// One step of the ring: issue the loads of a later k-tile into stage `wr`
// (when `load`) and multiply the k-tile held in stage `rd` into acc.  The two
// stages are disjoint; the restrict qualifiers tell the compiler so, and it
// then does not make the operand reads wait for the loads just issued (the
// caller's vmcnt wait and barrier order each stage's loads before its reads).
// CS: also add each B fragment's 8 values into cs[j] when do_cs (the column
// sums of B; see Epi2PartialCS).
template <int BM, int BN, int BK, bool A_KC, bool B_KC, int WGM, int WGN, bool CS = false>
__device__ __forceinline__ void g2_step(const char* __restrict__ rd, char* __restrict__ wr,
                                        bool load, const bf16_t* __restrict__ A, int lda,
                                        const bf16_t* __restrict__ Bm, int ldb, int m0, int n0,
                                        int M, int N, int kload, int kend, int wid, int lane,
                                        int wm, int wn,
                                        floatx16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                        const G2Off<BM, BK, A_KC, WGM * WGN>& pa,
                                        const G2Off<BN, BK, B_KC, WGM * WGN>& pb,
                                        bool do_cs = false, float* cs = nullptr) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr int kA = BM * BK * 2;
  if (load) {
    g2_issue<BM, BK, A_KC, NW>(A, lda, m0, M, kload, kend, wr, wid, lane, pa);
    g2_issue<BN, BK, B_KC, NW>(Bm, ldb, n0, N, kload, kend, wr + kA, wid, lane, pb);
  }
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 af[MT], bfr[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) af[i] = g2_frag<BM, BK, A_KC>(rd, wm * WTM + i * 32, kk, lane);
#pragma unroll
    for (int j = 0; j < NT; ++j) bfr[j] = g2_frag<BN, BK, B_KC>(rd + kA, wn * WTN + j * 32, kk, lane);
    if constexpr (CS) {
      if (do_cs) {
#pragma unroll
        for (int j = 0; j < NT; ++j) cs[j] += frag_sum8(bfr[j]);
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
  }
}

// Staged epilogue: bias (read from the tile's bias columns at LDS offset
// bias_off), activation and bf16 rounding into an LDS tile [BM][BN+8] that
// reuses the operand ring, then every 8 lanes store one 128-byte run of a row.
// Wave (wm, wn) holds the (BM/WGM) x (BN/WGN) sub-tile of D^T accumulators.
template <int BM, int BN, int WGM, int WGN, class Epi>
__device__ __forceinline__ void g2_store_staged(char* smem, int bias_off,
                                                const floatx16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                                const Epi& epi, int m0, int n0, int M, int N,
                                                int tid, int wm, int wn) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  const int lane = tid & 63;
  constexpr int SP = BN + 8;  // pitch (elements); 16-byte aligned rows
  bf16_t* ct = reinterpret_cast<bf16_t*>(smem);
  bar_nofence();  // every wave is done with the operand ring
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int cl = wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);  // local column
      const uint2 bu = *reinterpret_cast<const uint2*>(smem + bias_off + cl * 2);
      const float b[4] = {bf2f(bu.x & 0xffff), bf2f(bu.x >> 16), bf2f(bu.y & 0xffff),
                          bf2f(bu.y >> 16)};
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int rl = wm * WTM + i * 32 + (lane & 31);
        uint2 w;
        constexpr int ACT = ActOf<Epi>::value;
        w.x = pack_bf16x2(apply_act<ACT>(acc[i][j][4 * g] + b[0]),
                          apply_act<ACT>(acc[i][j][4 * g + 1] + b[1]));
        w.y = pack_bf16x2(apply_act<ACT>(acc[i][j][4 * g + 2] + b[2]),
                          apply_act<ACT>(acc[i][j][4 * g + 3] + b[3]));
        *reinterpret_cast<uint2*>(ct + rl * SP + cl) = w;
      }
    }
  bar_after_lds_writes();
  constexpr int kChunks = BM * BN / 8;
  static_assert(!Store8All<Epi>::value || kChunks % (64 * NW) == 0,
                "store8_all needs every lane in every pass");
  if constexpr (Store8All<Epi>::value) {
    // The epilogue's own operands (Epi::extra) of every pass are loaded first:
    // inside the store loop each load would wait behind the previous pass's
    // stores (they may alias), one memory latency per pass.
    constexpr int kPass = kChunks / (64 * NW);
    typename Epi::Extra ex[kPass];
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int c = tid + p * 64 * NW;
      const int m = m0 + c / (BN / 8), n = n0 + (c % (BN / 8)) * 8;
      ex[p] = epi.extra(m, n, m < M && n < N);
    }
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int c = tid + p * 64 * NW;
      const int rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
      const int m = m0 + rl, n = n0 + cl;
      epi.store8_all(m, n, *reinterpret_cast<const uint4*>(ct + rl * SP + cl), m < M && n < N,
                     lane, ex[p]);
    }
  } else {
    for (int c = tid; c < kChunks; c += 64 * NW) {
      const int rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
      const int m = m0 + rl, n = n0 + cl;
      if (m < M && n < N) epi.store8(m, n, *reinterpret_cast<const uint4*>(ct + rl * SP + cl));
    }
  }
}

// Staged epilogue in fp32 for kStagedF32 epilogues: for each wave row h of
// the WGM, the waves of that row write acc + bias (fp32) into an LDS tile
// [BM / WGM][BN + 4]; then all threads read 8-column runs (two 16-byte reads),
// with the epilogue's Extra8 of all passes loaded first, and call store8f.
template <int BM, int BN, int WGM, int WGN, class Epi>
__device__ __forceinline__ void g2_store_staged_f32(
    char* smem, int bias_off, const floatx16 (&acc)[BM / WGM / 32][BN / WGN / 32],
    const Epi& epi, int m0, int n0, int M, int N, int tid, int wm, int wn) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr int SP = BN + 4;                       // pitch (floats); 16-byte aligned rows
  constexpr int kChunks = WTM * BN / 8;            // 8-column runs of one wave row
  constexpr int kPass = (kChunks + 64 * NW - 1) / (64 * NW);
  const int lane = tid & 63;
  float* ct = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int h = 0; h < WGM; ++h) {
    bar_nofence();  // the ring (h = 0) or the previous half's runs are read
    if (wm == h) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cl = wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
          const uint2 bu = *reinterpret_cast<const uint2*>(smem + bias_off + cl * 2);
          const float b[4] = {bf2f(bu.x & 0xffff), bf2f(bu.x >> 16), bf2f(bu.y & 0xffff),
                              bf2f(bu.y >> 16)};
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const int rl = i * 32 + (lane & 31);
            *reinterpret_cast<float4*>(ct + rl * SP + cl) =
                make_float4(acc[i][j][4 * g] + b[0], acc[i][j][4 * g + 1] + b[1],
                            acc[i][j][4 * g + 2] + b[2], acc[i][j][4 * g + 3] + b[3]);
          }
        }
    }
    bar_after_lds_writes();
    typename Epi::Extra8 ex[kPass];
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int c = tid + p * 64 * NW;
      const int m = m0 + h * WTM + c / (BN / 8), n = n0 + (c % (BN / 8)) * 8;
      ex[p] = epi.extra8(m, n, c < kChunks && m < M && n < N);
    }
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int c = tid + p * 64 * NW;
      const int rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
      const int m = m0 + h * WTM + rl, n = n0 + cl;
      if (c < kChunks && m < M && n < N) {
        const float4 a = *reinterpret_cast<const float4*>(ct + rl * SP + cl);
        const float4 b = *reinterpret_cast<const float4*>(ct + rl * SP + cl + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        epi.store8f(m, n, v, ex[p]);
      }
    }
  }
}

// OCC: waves per SIMD the register allocation must allow (1 = no limit
// beyond the block size).
template <int BM, int BN, int BK, int NSTAGE, bool A_KC, bool B_KC, int WGM, int WGN, class Epi,
          int OCC = 1>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(OCC)))
void gemm2_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ Bm, int ldb, int M, int N,
    int K, int k_split, Epi epi) {
  constexpr int NW = WGM * WGN;
  using Cfg = Gemm2Cfg<BM, BN, BK, NSTAGE, A_KC, B_KC, NW>;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  // A staging epilogue reuses the ring's LDS, grown to the output tile when
  // that still fits the CU's 160 KB.
  constexpr int kEpiBytes = StagedF32<Epi>::value ? (BM / WGM) * (BN + 4) * 4
                            : Staged<Epi>::value   ? BM * (BN + 8) * 2
                                                   : 0;
  constexpr int kSmemAll =
      kEpiBytes > Cfg::kSmem && kEpiBytes + BN * 2 <= 160 * 1024 ? kEpiBytes : Cfg::kSmem;
  constexpr bool kStagedEpi = Staged<Epi>::value && kEpiBytes <= kSmemAll;
  // The staged epilogue reads the tile's bias columns from LDS, placed after
  // the ring / staging area.
  constexpr int kBiasOff = (kSmemAll + 15) / 16 * 16;
  constexpr int kLdsBytes = kStagedEpi ? kBiasOff + BN * 2 : kSmemAll;
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  __shared__ __align__(1024) char smem[kLdsBytes];

  const int tiles_n = (N + BN - 1) / BN;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  // Each XCD's run of consecutive tiles covers a band of row tiles; within
  // a band the order is column-major, so a band's A rows stay in that XCD's
  // L2 while the B columns stream through once.
  const int tiles_m = (M + BM - 1) / BM;
  const int band = max(1, tiles_m / 8);
  const int bi = tile / (band * tiles_n), loc = tile - bi * band * tiles_n;
  const int rows = min(band, tiles_m - bi * band);
  const int m0 = (bi * band + loc % rows) * BM, n0 = (loc / rows) * BN;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int kbeg = (int)blockIdx.y * k_split;
  const int kend = min(K, kbeg + k_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  floatx16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if constexpr (kStagedEpi) {
    // Bias columns n0 .. n0+BN-1 go straight to LDS (one 16-byte chunk per
    // lane of wave 0; chunks past N or a NULL bias read zeros).  Issued
    // before the ring, this load is older than every ring load of wave 0,
    // so the ring's vmcnt waits cover it; the barrier after the main loop
    // publishes it.
    static_assert(BN % 8 == 0 && BN / 8 <= 64, "bias tile");
    if (wid == 0 && lane < BN / 8) {
      const bf16_t* bp = epi.bias_ptr();
      const int n = n0 + 8 * lane;
      const bf16_t* g = (bp && n < N) ? bp + n : reinterpret_cast<const bf16_t*>(&g_zero16);
      __builtin_amdgcn_load_to_lds((void*)g, GA_LDS(smem + kBiasOff), 16, 0, 0);
    }
  }

  G2Off<BM, BK, A_KC, NW> pa;
  G2Off<BN, BK, B_KC, NW> pb;
  pa.init(lda, wid, lane);
  pb.init(ldb, wid, lane);
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < nk) {
      char* sa = smem + s * Cfg::kStage;
      g2_issue<BM, BK, A_KC, NW>(A, lda, m0, M, kbeg + s * BK, kend, sa, wid, lane, pa);
      g2_issue<BN, BK, B_KC, NW>(Bm, ldb, n0, N, kbeg + s * BK, kend, sa + Cfg::kA, wid, lane,
                                 pb);
    }

  // column sums of B (Epi2PartialCS): the first wave row of the first row
  // tile's blocks, from the B fragments it reads anyway
  constexpr bool kCS = ColSumB<Epi>::value;
  float cs[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) cs[j] = 0.f;
  bool do_cs = false;
  if constexpr (kCS) do_cs = epi.colsum && m0 == 0 && wm == 0;

  for (int kt = 0; kt < nk; ++kt) {
    // tile kt is complete once at most (later tiles issued) x loads remain
    const int later = min(nk - 1, kt + NSTAGE - 2) - kt;
    if (later >= NSTAGE - 2) wait_vmcnt<Cfg::kLoads * (NSTAGE - 2)>();
    else if (NSTAGE > 3 && later == 2) wait_vmcnt<Cfg::kLoads * 2>();
    else if (later == 1) wait_vmcnt<Cfg::kLoads>();
    else wait_vmcnt<0>();
    bar_nofence();
    const int kn = kt + NSTAGE - 1;
    g2_step<BM, BN, BK, A_KC, B_KC, WGM, WGN, kCS>(
        smem + (kt % NSTAGE) * Cfg::kStage, smem + (kn % NSTAGE) * Cfg::kStage, kn < nk, A, lda,
        Bm, ldb, m0, n0, M, N, kbeg + kn * BK, kend, wid, lane, wm, wn, acc, pa, pb, do_cs, cs);
  }
  if constexpr (kCS) {
    // lanes l and l ^ 32 hold the two k halves of column l % 32 of each
    // fragment: B fragment j of wave column wn covers columns
    // n0 + wn * WTN + 32 j + (lane % 32)
    if (do_cs) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float v = cs[j] + __shfl_xor(cs[j], 32);
        const int n = n0 + wn * WTN + j * 32 + lane;
        if (lane < 32 && n < N) epi.store_colsum(n, v);
      }
    }
  }

  if constexpr (kStagedEpi) {
    if constexpr (StagedF32<Epi>::value)
      g2_store_staged_f32<BM, BN, WGM, WGN>(smem, kBiasOff, acc, epi, m0, n0, M, N, tid, wm, wn);
    else
      g2_store_staged<BM, BN, WGM, WGN>(smem, kBiasOff, acc, epi, m0, n0, M, N, tid, wm, wn);
  } else {
    static_assert(!Store8All<Epi>::value, "store8_all epilogues need the staged path");
    // ---- epilogue straight from the D^T accumulators
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + wm * WTM + i * 32 + (lane & 31);
      if (m >= M) continue;
      if constexpr (SplitOffsets<Epi>::value) {
        const size_t ro = epi.row_off(m);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int nb = n0 + wn * WTN + j * 32;
          if (nb >= N) continue;
          const size_t co = epi.col_off(nb);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dn = 8 * g + 4 * (lane >> 5);
            const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                acc[i][j][4 * g + 3]};
            epi.store(ro + co + dn, nb + dn, v);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
            if (n < N) {
              const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                  acc[i][j][4 * g + 3]};
              epi(m, n, v);
            }
          }
      }
    }
  }
}

// splits > 1 divides K into that many slices (multiples of BK); returns the
// number of slices launched.
template <int BM, int BN, int NSTAGE, int BK, int WGM, int WGN, bool A_KC, bool B_KC,
          int OCC = 1, class Epi>
inline int launch_gemm2(const bf16_t* A, int lda, const bf16_t* B, int ldb, int M, int N,
                        int K, const Epi& epi, hipStream_t st, int splits = 1) {
  const int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (grid == 0 || K <= 0) return 0;
  if (splits < 1) splits = 1;
  int k_split = (K + splits - 1) / splits;
  k_split = (k_split + BK - 1) / BK * BK;
  const int ns = (K + k_split - 1) / k_split;
  hipLaunchKernelGGL((gemm2_kernel<BM, BN, BK, NSTAGE, A_KC, B_KC, WGM, WGN, Epi, OCC>),
                     dim3(grid, ns), dim3(64 * WGM * WGN), 0, st, A, lda, B, ldb, M, N, K,
                     k_split, epi);
  return ns;
}

}  // namespace gpt_attn
