// handle.cuh -- the layer handle, its workspace layout and host helpers
// shared by the translation units of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <math.h>

#include "../../include/gpt_attn.h"
#include "philox.cuh"

// Tile shapes (BM, BN, pipeline stages, BK, wave grid rows, wave grid columns)
// of the bf16 GEMMs.
// c_attn: 256 x 256 tiles over 16 waves (4 x 4 grid of 64 x 64 wave tiles,
// 126 VGPRs), so each SIMD holds four waves of the block instead of two and
// the operand loads of some waves are issued while others multiply
#ifndef GA_QKV_TILE
#define GA_QKV_TILE 256, 256, 2, 64, 4, 4
#endif
#ifndef GA_QKV_OCC
#define GA_QKV_OCC 4
#endif
#ifndef GA_PROJ_TILE
#define GA_PROJ_TILE 192, 256, 2, 64, 2, 4
#endif
#ifndef GA_DGRAD_TILE
#define GA_DGRAD_TILE 192, 256, 2, 64, 2, 4
#endif
// Projections onto C columns with C a multiple of 384 and at least 128 such
// tiles: the GEMM whose loader and MFMA waves sit on separate SIMDs
// (gemm3.cuh), 96 x 384 tiles (BM, BN, stages, BK, wave grid of six):
// the forward c_proj (K = C) and the dx product of the backward (K = 3C).
#ifndef GA_PROJ3_TILE
#define GA_PROJ3_TILE 96, 384, 4, 32, 1, 6
#endif
#ifndef GA_DGRAD3_TILE
#define GA_DGRAD3_TILE 96, 384, 2, 64, 1, 6
#endif
#ifndef GA_ATTN_STAGES
#define GA_ATTN_STAGES 2
#endif
#ifndef GA_WGRAD_TILE
#define GA_WGRAD_TILE 128, 128, 2, 64, 2, 2
#endif
// weight gradient of c_attn (C x 3C over all B*T rows): 256 x 128 tiles split
// along the rows to about one block per CU (4 slices at C = 768: half the
// fp32 partials that 256 x 256 tiles in 8 slices leave for the reduction),
// 16 waves of 64 x 32 (four waves per SIMD, as c_attn)
#ifndef GA_WGRAD_ATTN_TILE
#define GA_WGRAD_ATTN_TILE 256, 128, 2, 64, 4, 4
#endif
#ifndef GA_WGRAD_ATTN_PER_CU
#define GA_WGRAD_ATTN_PER_CU 1
#endif
// MLP: c_fc [C -> 4C] with the GELU epilogue (12 waves of 64 x 96, three per
// SIMD), c_proj [4C -> C] (waves per SIMD as the last value).
#ifndef GA_FC_TILE
#define GA_FC_TILE 192, 384, 2, 64, 3, 4, true, false, 1
#endif
#ifndef GA_FCPROJ_TILE
#define GA_FCPROJ_TILE 192, 256, 2, 64, 2, 4, true, false, 1
#endif


struct gpt_attn_handle {
  int C, H, hs, max_B, max_T, dtype;
  int device;
  size_t esize;  // bytes per element
  char* ws;      // one allocation, carved below
  size_t ws_bytes;
  // carved regions
  void* qkv;     // [3][B][H][T][hs]
  void* o;       // [B][T][C]
  float* lse;    // [B][H][T]
  void* dym;     // [B][T][C]     backward: gradient of merged heads
  void* dqkv;    // [B][T][3C]    backward: gradient of c_attn output
  float* delta;  // [B][H][T]     backward: rowsum(dO * O)
  float* part;   // split-K partial sums of weight gradients (fp32)
  void* ln;      // [B][T][C]     Pre-LN block: ln_1 of the input
  float* rowstats;  // backward: L (log2 units) and D per softmax row, rows of
                    // T rounded up to 64: [2][B][H][Tpad]
  unsigned* counters;  // [kCounters] arrival counters of kernels whose last
                       // block finishes the work of the others; zero between
                       // launches (set at creation, reset by that last block)
  size_t part_elems;
  // state of the last forward
  int saved, saved_B, saved_T;
  // q/k/v of the last forward (any kind) still in the workspace: B, T
  int last_B, last_T;
  // dropout rate and generator seed of later forwards (0: none); the rate
  // and seed of the saved forward
  float drop_p;
  unsigned long long drop_seed;
  float saved_drop_p;
  unsigned long long saved_drop_seed;
  // keep bits of the attention-weight dropout (keep_bits.cuh) stored by a
  // forward that keeps state, read by the backward; allocated when dropout
  // is first switched on, sized for max_B and max_T
  uint32_t* keepq;
  uint16_t* keepk;
  // optional stage events (measurement hook)
  hipEvent_t ev[8];
  int n_ev;
  // second stream of the backward (default priority, non-blocking): the
  // c_proj weight and bias gradients run there beside the data-gradient
  // chain, forked from and joined back into the caller's stream by these
  // events
  hipStream_t side;
  hipEvent_t ev_fork, ev_join;
};

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Upper bound on the split-K slices of the weight-gradient GEMMs, and the
// number of row slices of the bias-gradient column sums.
constexpr int kWgradSplits = 8;
constexpr int kColsumSplits = 64;
constexpr int kCounters = 4096;

int check_dims(int C, int n_head, int max_B, int max_T, int dtype) {
  if (C <= 0 || n_head <= 0 || max_B <= 0 || max_T <= 0) return GPT_ATTN_ERR_INVALID_ARG;
  if (dtype != GPT_ATTN_F32 && dtype != GPT_ATTN_BF16) return GPT_ATTN_ERR_INVALID_ARG;
  if (C % n_head != 0) return GPT_ATTN_ERR_SHAPE;
  const int hs = C / n_head;
  if (hs != 32 && hs != 64) return GPT_ATTN_ERR_UNSUPPORTED;
  // every index below fits in 32 bits per tensor row count / 64-bit offsets
  if ((long long)max_B * max_T > (1LL << 30)) return GPT_ATTN_ERR_SHAPE;
  return GPT_ATTN_OK;
}

struct Layout {
  size_t qkv, o, lse, dym, dqkv, delta, part, ln, rowstats, counters, total, part_elems;
};

Layout layout(int C, int H, int max_B, int max_T, size_t es) {
  Layout L;
  const size_t BT = (size_t)max_B * max_T;
  size_t off = 0;
  L.qkv = off;   off = align_up(off + 3 * BT * C * es);
  L.o = off;     off = align_up(off + BT * C * es);
  L.lse = off;   off = align_up(off + (size_t)max_B * H * max_T * sizeof(float));
  L.dym = off;   off = align_up(off + BT * C * es);
  L.dqkv = off;  off = align_up(off + 3 * BT * C * es);
  L.delta = off; off = align_up(off + (size_t)max_B * H * max_T * sizeof(float));
  // split-K partials of the weight gradients, each slice C + 1 rows (the last
  // holds the bias gradient's column sums), then column-sum partials
  L.part_elems = (size_t)kWgradSplits * (C + 1) * 3 * C + (size_t)kColsumSplits * 3 * C;
  L.part = off;  off = align_up(off + L.part_elems * sizeof(float));
  L.ln = off;    off = align_up(off + BT * C * es);
  L.rowstats = off;
  off = align_up(off + 2 * (size_t)max_B * H * ((max_T + 63) / 64 * 64) * sizeof(float));
  L.counters = off;
  off = align_up(off + kCounters * sizeof(unsigned));
  L.total = off;
  return L;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline void mark(const gpt_attn_handle* h, int i, hipStream_t st) {
  if (i < h->n_ev) (void)hipEventRecord(h->ev[i], st);
}

// Dropout parameters of rate p and seed (philox.cuh).
inline gpt_attn::DropParams make_drop(float p, unsigned long long seed) {
  const double t = floor((double)p * 4294967296.0);
  gpt_attn::DropParams d;
  d.k0 = (uint32_t)seed;
  d.k1 = (uint32_t)(seed >> 32);
  d.thresh = t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
  const double t16 = floor((double)p * 65536.0);
  d.thresh16 = t16 >= 65535.0 ? 0xFFFFu : (uint32_t)t16;
  d.scale = (float)(1.0 / (1.0 - (double)p));
  return d;
}

inline int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GPT_ATTN_OK : GPT_ATTN_ERR_HIP;
}

}  // namespace

