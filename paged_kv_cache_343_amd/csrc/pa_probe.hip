// Measurement aid, not part of the decode path: a streaming HBM read whose
// rate is the practical ceiling the decode kernels are compared against.
// Each thread reads 16-byte words with a grid-sized stride and folds them
// into a value that is stored only if it matches a sentinel, so the reads
// cannot be dropped and nothing but the reads touches memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_probe.h"

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n,
                                                          uint32_t* sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = p[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

extern "C" int pa_probe_stream_read(const void* buf, size_t bytes, int workgroups, void* sink,
                                    void* stream) {
  if (!buf || !sink || bytes < 16 || workgroups <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
