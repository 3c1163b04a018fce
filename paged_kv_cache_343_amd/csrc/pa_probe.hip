// Measurement aid, not part of the decode path: streaming HBM reads whose
// best rate over a sweep of launch shapes and access patterns is the
// practical ceiling the decode kernels are compared against.
//
// Patterns (U = 16-byte loads in flight per lane, issued back to back before
// any is used; plain or streaming (non-temporal) cache policy):
//   0 grid-stride: thread t of T reads words t, t + T, t + 2T, ..., so each
//     wave load covers 1 KiB of consecutive bytes (whole 128-byte lines);
//   1 wave tiles: each wave reads U KiB of consecutive bytes per iteration,
//     the waves taking consecutive tiles in turn;
//   2 random 4 KiB tiles: the buffer's two halves stand for a K and a V
//     pool; per iteration a wave reads one 4 KiB tile of each half at the
//     same pseudo-random tile index (a bijective hash of the iteration and
//     wave), the gather that paged decode makes (U = 8: both tiles' loads in
//     flight together).
// The words are folded into a value that is stored only if it matches a
// sentinel, so the reads cannot be dropped and nothing but the reads touches
// memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4_t ld(const u32x4_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

__device__ __forceinline__ uint32_t fold(const u32x4_t& v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int U, bool NT>
__global__ __launch_bounds__(256) void grid_stride_kernel(const u32x4_t* __restrict__ p,
                                                          size_t n, uint32_t* sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld<NT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= fold(v[u]);
  }
  for (; i < n; i += stride) x ^= fold(p[i]);
  if (x == 0x9e3779b9u) sink[0] = x;
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void wave_tile_kernel(const u32x4_t* __restrict__ p, size_t n,
                                                        uint32_t* sink) {
  uint32_t x = 0;
  const size_t lane = threadIdx.x & 63;
  const size_t wave = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const size_t waves = ((size_t)gridDim.x * blockDim.x) >> 6;
  const size_t tile = (size_t)U * 64;                  // words per wave per iteration
  const size_t ntiles = n / tile;
  for (size_t t = wave; t < ntiles; t += waves) {
    const u32x4_t* b = p + t * tile + lane;
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld<NT>(b + u * 64);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= fold(v[u]);
  }
  for (size_t i = ntiles * tile + wave * 64 + lane; i < n; i += waves * 64) x ^= fold(p[i]);
  if (x == 0x9e3779b9u) sink[0] = x;
}

// Random 4 KiB tiles (256 words) of the two halves. The tile count per half
// is rounded down to a power of two so that k -> (k * odd) mod count is a
// bijection; iteration k of wave w reads tile hash(k * waves + w).
template <int U, bool NT>
__global__ __launch_bounds__(256) void random_tile_kernel(const u32x4_t* __restrict__ p,
                                                          size_t n, uint32_t* sink) {
  static_assert(U == 4 || U == 8, "one or two 4 KiB tiles in flight");
  uint32_t x = 0;
  const size_t lane = threadIdx.x & 63;
  const size_t wave = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const size_t waves = ((size_t)gridDim.x * blockDim.x) >> 6;
  const size_t half = n / 2;
  size_t count = 1;
  while (count * 2 * 256 <= half) count *= 2;
  const u32x4_t* kp = p;
  const u32x4_t* vp = p + half;
  for (size_t k = wave; k < count; k += waves) {
    const size_t t = (k * 0x9E3779B1ull) & (count - 1);
    const u32x4_t* kb = kp + t * 256 + lane;
    const u32x4_t* vb = vp + t * 256 + lane;
    if constexpr (U == 8) {
      u32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = ld<NT>(kb + u * 64);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[4 + u] = ld<NT>(vb + u * 64);
#pragma unroll
      for (int u = 0; u < 8; ++u) x ^= fold(v[u]);
    } else {
      u32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = ld<NT>(kb + u * 64);
#pragma unroll
      for (int u = 0; u < 4; ++u) x ^= fold(v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = ld<NT>(vb + u * 64);
#pragma unroll
      for (int u = 0; u < 4; ++u) x ^= fold(v[u]);
    }
  }
  if (x == 0x9e3779b9u) sink[0] = x;
}

using ProbeKernel = void (*)(const u32x4_t*, size_t, uint32_t*);

template <bool NT>
ProbeKernel pick(int pattern, int loads) {
  switch (pattern * 16 + loads) {
    case 0 * 16 + 1: return grid_stride_kernel<1, NT>;
    case 0 * 16 + 2: return grid_stride_kernel<2, NT>;
    case 0 * 16 + 4: return grid_stride_kernel<4, NT>;
    case 0 * 16 + 8: return grid_stride_kernel<8, NT>;
    case 1 * 16 + 1: return wave_tile_kernel<1, NT>;
    case 1 * 16 + 2: return wave_tile_kernel<2, NT>;
    case 1 * 16 + 4: return wave_tile_kernel<4, NT>;
    case 1 * 16 + 8: return wave_tile_kernel<8, NT>;
    case 2 * 16 + 4: return random_tile_kernel<4, NT>;
    case 2 * 16 + 8: return random_tile_kernel<8, NT>;
    default: return nullptr;
  }
}

}  // namespace

extern "C" int pa_probe_stream_read(const void* buf, size_t bytes, int workgroups,
                                    int loads_per_lane, int nontemporal, int pattern,
                                    void* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || workgroups <= 0 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return 1;
  if (pattern == 2 && bytes < 2 * 4096) return 1;
  const ProbeKernel kern =
      nontemporal ? pick<true>(pattern, loads_per_lane) : pick<false>(pattern, loads_per_lane);
  if (!kern) return 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(buf),
                     bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
