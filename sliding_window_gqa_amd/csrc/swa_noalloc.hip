// swa_noalloc.hip — swa_decode_step for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): the split-K partial results go to a fixed device array
// of this library instead of a caller workspace.
//
// The array lives for the life of the process on every GPU the library runs
// on (each GPU holds its own copy at its own address).  Its device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and only that address is handed to kernels; the array's name is a
// host-side stand-in, not a device address.  Nothing here allocates.
//
// Every call on one GPU shares that GPU's array: calls that overlap in time
// on one GPU (different streams, or threads) race on it and must not be
// issued.  No part of the array needs to start at zero: the decode kernel
// writes every split's partial before the combine pass reads it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/swa.h"

// The array itself, one copy per device (zero-filled at load).
static __device__ __attribute__((aligned(256))) unsigned char scratch[4u << 20];

namespace {

constexpr size_t kScratchBytes = sizeof(scratch);

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, or null

// Device address of this device's copy of the array (null on failure).
void* scratch_address(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t swa_noalloc_scratch_bytes(void) { return kScratchBytes; }

int swa_decode_step_noalloc(const swa_params* params, const void* q, const void* k, const void* v,
                            void* k_cache, void* v_cache, const int32_t* pos, void* out, float* lse,
                            hipStream_t stream) {
  // the argument checks of swa_decode_step, before any HIP call
  const size_t need = swa_decode_workspace_bytes(params);
  if (need == 0) {
    const int st = swa_decode_step(params, q, k, v, k_cache, v_cache, pos, out, lse, nullptr, 0, stream);
    return st != SWA_OK ? st : SWA_ERR_SHAPE;
  }
  if (!q || !k || !v || !k_cache || !v_cache || !pos || !out) return SWA_ERR_NULL;
  if (need > kScratchBytes) return SWA_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SWA_ERR_LAUNCH;
  void* ws = scratch_address(dev);
  if (!ws) return SWA_ERR_LAUNCH;
  return swa_decode_step(params, q, k, v, k_cache, v_cache, pos, out, lse, ws, kScratchBytes, stream);
}

}  // extern "C"
