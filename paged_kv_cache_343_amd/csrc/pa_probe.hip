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
//
// A second probe times how far matrix-core and vector work overlap on one
// SIMD: workgroups of 8 waves repeat, per iteration, 16 independent
// v_mfma_f32_16x16x32_bf16 (four accumulators) and/or 64 dependent-in-eights
// fp32 FMAs, in these modes:
//   0 MFMAs only; 1 FMAs only; 2 both in every wave, interleaved;
//   3 waves 0-3 MFMAs and waves 4-7 FMAs (one of each kind per SIMD);
//   4 MFMAs only, one dependent chain; 5 16 exp2 per iteration only.
// Each thread stores one float at the end; nothing else touches memory.
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(512) void overlap_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(lane * 0.001f + i);
    b[i] = (__bf16)(w * 0.01f + i * 0.5f);
  }
  f32x4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = lane * 0.01f + i;
  const bool do_m = MODE == 0 || MODE == 4 || (MODE == 3 && w < 4);
  const bool do_v = MODE == 1 || (MODE == 3 && w >= 4);
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 2) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        acc[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j & 3], 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) x[(4 * j + v) & 7] = fmaf(x[(4 * j + v) & 7], 1.0001f, 0.5f);
      }
    } else {
      if (do_m) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int k = MODE == 4 ? 0 : (j & 3);
          acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
        }
      }
      if (do_v) {
#pragma unroll
        for (int v = 0; v < 64; ++v) x[v & 7] = fmaf(x[v & 7], 1.0001f, 0.5f);
      }
      if constexpr (MODE == 5) {
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v & 7] = __builtin_amdgcn_exp2f(x[v & 7]);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = s;
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

// out: workgroups * 512 floats.
extern "C" int pa_probe_mfma_valu(int mode, int workgroups, int iters, float* out, void* stream) {
  if (!out || workgroups <= 0 || iters <= 0) return 1;
  void (*kern)(float*, int) = nullptr;
  switch (mode) {
    case 0: kern = overlap_kernel<0>; break;
    case 1: kern = overlap_kernel<1>; break;
    case 2: kern = overlap_kernel<2>; break;
    case 3: kern = overlap_kernel<3>; break;
    case 4: kern = overlap_kernel<4>; break;
    case 5: kern = overlap_kernel<5>; break;
    default: return 1;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)workgroups), dim3(512), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
