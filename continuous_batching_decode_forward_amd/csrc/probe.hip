// probe.hip -- a streaming-read probe of the device's HBM: the bandwidth a
// plain read of a large buffer reaches on this device, measured beside the
// step's kernels so that their rooflines can be read against what the
// memory system delivers as well as against its published peak. Not part
// of the step.
//
// Every thread of the grid (blocks x 1024) reads 16-byte words i = tid,
// tid + G, tid + 2G, ... (G threads in all) with the non-temporal hint, so
// each wave's load covers 1 KB of consecutive bytes and the grid sweeps the
// buffer front to back; the words are folded by XOR into one value per
// thread, which is stored so that no load can be dropped. (On MI355X the
// best of 512-8192 blocks of 256-1024 threads and 1, 4 or 8 loads in
// flight per thread was 512 x 1024 threads with one load per turn.)
#include "common.h"
#include "kernels.h"

namespace cbd {

#define PROBE_THREADS 1024

__global__ __launch_bounds__(PROBE_THREADS) void read_probe_kernel(const uint16_t* __restrict__ p,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ out) {
  const size_t tid = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
  const size_t G = (size_t)gridDim.x * PROBE_THREADS;
  uint32_t acc = 0;
  for (size_t i = tid; i < n16; i += G) {
    const uint4 v = load_stream16(p + 8 * i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[tid] = acc;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, int32_t blocks,
                             hipStream_t st) {
  read_probe_kernel<<<blocks, PROBE_THREADS, 0, st>>>(static_cast<const uint16_t*>(buf), bytes / 16,
                                                      out);
  return hipGetLastError();
}

}  // namespace cbd
