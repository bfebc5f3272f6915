// sampler_noalloc.hip -- the batched sampler's row scratch as a fixed device
// array, for callers that cannot allocate device memory (code under graph
// capture, tight serving loops): cbd_sample_logits_noalloc runs the same
// sampler kernels as cbd_sample_logits, with the rows that do not fit on
// chip (vocabularies above 65536) staged here instead of in the engine's
// workspace.
//
// Every call on one GPU shares that GPU's copy of the array and leaves its
// contents behind; the sampler writes every scratch value of a row before it
// reads it, so nothing needs clearing between calls. Calls that overlap on
// one GPU (two streams, two threads) race on the array.
#include <mutex>

#include "kernels.h"

namespace cbd {

#define NOALLOC_SCRATCH_FLOATS (4u << 20)  // 16 MiB per device
#define NOALLOC_MAX_DEVICES 64

static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_FLOATS];

static std::mutex g_noalloc_mu;
static float* g_noalloc_ptr[NOALLOC_MAX_DEVICES];

// The device address of the current device's scratch array, looked up once
// per device with that device current (the array's host-side name is a
// stand-in, never a device address).
hipError_t noalloc_scratch(float** ptr, size_t* floats) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_noalloc_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_noalloc_ptr[dev];
  *floats = NOALLOC_SCRATCH_FLOATS;
  return hipSuccess;
}

}  // namespace cbd
