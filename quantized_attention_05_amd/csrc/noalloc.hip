// sattn_fwd_noalloc: the drop-in self-attention of sattn_fwd with its workspace taken from a fixed device array of
// the library instead of the caller, for callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid allocation).  The array is a file-scope __device__ object: every GPU the
// library runs on holds its own copy, of kNoAllocBytes, until the process ends.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "sattn_internal.h"

namespace {

constexpr size_t kNoAllocBytes = SATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// In host code this name is only a handle for hipGetSymbolAddress: the device address of each GPU's copy is looked
// up once per device and used everywhere instead.
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of the current device's copy of `scratch` (nullptr if it cannot be resolved).  Resolved once
// per device, with that device current, then kept.
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" sattn_status sattn_fwd_noalloc(const sattn_tensor* q, const sattn_tensor* k, const sattn_tensor* v,
                                          const sattn_tensor* o, float sm_scale, int mode, int blk_q, int blk_k,
                                          sattn_stream_t stream) {
  if (!q || !k) return SATTN_ERR_INVALID_ARG;
  const size_t need = sattn_workspace_bytes(q->B, q->H, q->N, k->N, q->d, blk_q, blk_k, mode);
  // an invalid shape (need == 0) falls through to sattn_fwd's own checks and their status
  if (need > kNoAllocBytes) return SATTN_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SATTN_ERR_HIP;
  void* ws = device_scratch(dev);
  if (!ws) return SATTN_ERR_HIP;
  return sattn_fwd(q, k, v, o, sm_scale, mode, blk_q, blk_k, ws, kNoAllocBytes, stream);
}
