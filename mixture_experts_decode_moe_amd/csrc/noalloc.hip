// The layer entry point for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): moe_layer_forward_noalloc runs moe_layer_forward_ex with its
// workspace in this file's device array instead of a caller's buffer.
//
// The array lives in every GPU the library runs on, from the module's load
// until the process ends.  Host code never uses the array's name as an
// address (on the host it names a stand-in, not device memory): the first
// call on a device, with that device current, asks the runtime for the
// device address once and keeps it per device.
#include <stdlib.h>

#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch array (nullptr on failure).
// Also clears the array's control words once, on the stream of the first
// call (every call leaves them zero again).
void *device_scratch(hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    if (moe_workspace_init(p, kScratchBytes, s) != MOE_OK) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const moe_layer *L, const uint16_t *x_bf16, int32_t T, float *y,
                                         const moe_residual *res, int32_t *topk_ids, float *topk_w,
                                         const moe_forward_opts *opts, void *stream) {
  const size_t need = T > 0 ? moe_workspace_bytes(L, T) : 0;
  // invalid layers and token counts, and calls without tokens: the same
  // validation and status as the workspace entry point, which launches
  // nothing for them (and no device is touched)
  if (need == 0) return moe_layer_forward_ex(L, x_bf16, T, y, res, topk_ids, topk_w, nullptr, 0, opts, stream);
  if (need > kScratchBytes) return MOE_ERR_UNSUPPORTED;  // beyond the fixed scratch array
  hipStream_t s = static_cast<hipStream_t>(stream);
  void *ws = device_scratch(s);
  if (!ws) return MOE_ERR_HIP;
  // The prefill gate/up item queue (the control words) must be zero when a
  // call starts; every call leaves it zero, and calls that can take the
  // prefill family clear it anyway with a fill kernel (no memset node, so
  // the call stays capturable).
  const bool may_prefill = T > moe::kFusedTokens || (opts && opts->path == MOE_PATH_PREFILL) || getenv("MOE_FORCE_PATH");
  if (may_prefill && T > 0) {
    const int rc = moe_workspace_init(ws, kScratchBytes, stream);
    if (rc != MOE_OK) return rc;
  }
  return moe_layer_forward_ex(L, x_bf16, T, y, res, topk_ids, topk_w, ws, kScratchBytes, opts, stream);
}
