// gpt_noalloc.hip -- the allocation-free forward (include/gpt_attn.h,
// gpt_attn_forward_noalloc).
//
// Same launch sequence and kernels as gpt_attn_forward on a bf16 handle
// (layer_fwd.cuh), without a handle: the intermediates -- q, k, v
// head-major, the merged heads and, for short sequences, the split-K partial
// sums -- live in `scratch`, a file-scope device array that each GPU holds
// from the first call on it until the process ends.  In host code the name
// `scratch` is only a host-side stand-in for the array: kernels receive the
// device address that hipGetSymbolAddress returns for the current device,
// looked up once per device and kept in g_scratch.  No call here allocates
// device memory.
#include <mutex>

#include "handle.cuh"
#include "layer_fwd.cuh"

using namespace gpt_attn;

static __device__ __align__(256) char scratch[GPT_ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices];  // device address of `scratch` on each device

// The current device's copy of `scratch` (first call on a device: look it
// up with that device current).
int scratch_on_current_device(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GPT_ATTN_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return GPT_ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return GPT_ATTN_ERR_HIP;
    }
    g_scratch[dev] = (char*)p;
  }
  *out = g_scratch[dev];
  return GPT_ATTN_OK;
}

}  // namespace

extern "C" int gpt_attn_forward_noalloc(const void* x, int B, int T, int C, int n_head,
                                        const void* W_attn, const void* b_attn,
                                        const void* W_proj, const void* b_proj, void* y,
                                        void* stream) {
  // ---- validation (host only)
  if (!x || !W_attn || !W_proj || !y) return GPT_ATTN_ERR_INVALID_ARG;
  if (B < 0 || T < 0) return GPT_ATTN_ERR_INVALID_ARG;
  int rc = check_dims(C, n_head, B > 0 ? B : 1, T > 0 ? T : 1, GPT_ATTN_BF16);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(W_attn) || !aligned16(W_proj) || !aligned16(y) ||
      (b_attn && !aligned16(b_attn)) || (b_proj && !aligned16(b_proj)))
    return GPT_ATTN_ERR_ALIGN;
  if (B == 0 || T == 0) return GPT_ATTN_OK;
  const size_t M = (size_t)B * T;
  const size_t qkv_bytes = align_up(3 * M * C * sizeof(bf16_t));
  const size_t o_bytes = align_up(M * C * sizeof(bf16_t));
  if (qkv_bytes + o_bytes > (size_t)GPT_ATTN_NOALLOC_SCRATCH_BYTES) return GPT_ATTN_ERR_SHAPE;
  char* base = nullptr;
  rc = scratch_on_current_device(&base);
  if (rc) return rc;

  // A host-side description of the scratch regions in the layout the launch
  // sequence reads from a handle (nothing is allocated; no stage events).
  gpt_attn_handle view{};
  view.C = C;
  view.H = n_head;
  view.hs = C / n_head;
  view.max_B = B;
  view.max_T = T;
  view.dtype = GPT_ATTN_BF16;
  view.esize = sizeof(bf16_t);
  view.qkv = base;
  view.o = base + qkv_bytes;
  view.part = (float*)(base + qkv_bytes + o_bytes);
  view.part_elems = ((size_t)GPT_ATTN_NOALLOC_SCRATCH_BYTES - qkv_bytes - o_bytes) / sizeof(float);
  layer_forward_bf16(&view, (const bf16_t*)x, B, T, (const bf16_t*)W_attn,
                     (const bf16_t*)b_attn, (const bf16_t*)W_proj, (const bf16_t*)b_proj,
                     (bf16_t*)y, nullptr, nullptr, as_stream(stream));
  return launch_status();
}
