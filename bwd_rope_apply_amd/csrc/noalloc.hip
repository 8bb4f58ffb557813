// The forward pass for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops): its workspace is a fixed-size
// file-scope device array, one copy per GPU, instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "rope_attn.h"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)ROPE_ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

// The forward's workspace on every GPU the library runs on (held until the
// process ends).  In host code this name is a stand-in, not a device
// address: only the per-device address from hipGetSymbolAddress is passed
// to kernels.
__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_lock;
void* g_addr[MAX_DEVICES] = {};

// This device's address of `scratch`, looked up once per device (with that
// device current, as it is for the calling thread), or null on failure.
void* scratch_on(int dev) {
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_addr[dev] = ptr;
  }
  return g_addr[dev];
}

}  // namespace

extern "C" int rope_attn_fwd_noalloc(const void* q, const void* k, const void* v, float* o,
                                     float* lse, int B, int H, int N, int D, int dtype, double base,
                                     const float* alpha, int causal, void* stream) {
  const size_t need = rope_attn_fwd_workspace_bytes(B, H, N, D, dtype, causal);
  const auto bad_ptr = [](const void* p) { return !p || ((uintptr_t)p & 15u) != 0; };
  if (need == 0 || bad_ptr(q) || bad_ptr(k) || bad_ptr(v) || bad_ptr(o) || bad_ptr(lse) ||
      ((uintptr_t)alpha & 15u) != 0 || !(base > 0.0) || !isfinite(base) ||
      (causal != 0 && causal != 1))
    // invalid arguments: the forward's own validation names them (before any HIP call)
    return rope_attn_fwd_ex(ROPE_ATTN_STAGE_ALL, nullptr, q, k, v, o, lse, B, H, N, D, dtype, base,
                            alpha, causal, nullptr, 0, stream);
  if (need > SCRATCH_BYTES) return ROPE_ATTN_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return ROPE_ATTN_ERR_HIP;
  void* ws = scratch_on(dev);
  if (!ws) return ROPE_ATTN_ERR_HIP;
  return rope_attn_fwd_ex(ROPE_ATTN_STAGE_ALL, nullptr, q, k, v, o, lse, B, H, N, D, dtype, base,
                          alpha, causal, ws, SCRATCH_BYTES, stream);
}
