// Measurement aid, not part of the decode path: a streaming HBM read whose
// best rate over a sweep of launch shapes is the practical ceiling the
// decode kernels are compared against.
//
// Thread t of a grid of T threads reads the 16-byte words t, t + T, t + 2T,
// ... (each wave's load covers 1 KiB of consecutive bytes: whole 128-byte
// lines), U of them issued back to back before any is used, so U loads of
// 16 bytes per lane are in flight at once (U = 1, 2, 4 or 8), with either the
// plain or the streaming (non-temporal) cache policy. The words are folded
// into a value that is stored only if it matches a sentinel, so the reads
// cannot be dropped and nothing but the reads touches memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, size_t n,
                                                          uint32_t* sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4_t v = p[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9e3779b9u) sink[0] = x;
}

template <bool NT>
void (*pick(int loads))(const u32x4_t*, size_t, uint32_t*) {
  switch (loads) {
    case 1: return stream_read_kernel<1, NT>;
    case 2: return stream_read_kernel<2, NT>;
    case 4: return stream_read_kernel<4, NT>;
    case 8: return stream_read_kernel<8, NT>;
    default: return nullptr;
  }
}

}  // namespace

extern "C" int pa_probe_stream_read(const void* buf, size_t bytes, int workgroups,
                                    int loads_per_lane, int nontemporal, void* sink,
                                    void* stream) {
  if (!buf || !sink || bytes < 16 || workgroups <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return 1;
  auto kern = nontemporal ? pick<true>(loads_per_lane) : pick<false>(loads_per_lane);
  if (!kern) return 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(buf), bytes / 16,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
