// gfx950 kernels for paged decode attention, the slot write and the block
// copy.
//
// The decode computes, for every sequence i and query head h (KV head
// g = h / G), softmax-weighted V over the positions p < seq_len[i], where
// position p lives in physical block block_tables[i][p / bs] at offset
// p % bs (the per-position lookup of the single decode step pseudo-code on
// the zenaique.com page "Walk through paged attention end to end ..."; the
// attention itself is ordinary attention, as its "Red flags" section
// stresses). Tokens of one head are contiguous inside a block ("PagedAttention
// & vLLM", "The insight: KV cache as virtual memory"; n4n.ai "How
// PagedAttention works"), so each block is one contiguous bs x D tile per
// head and is read with full 16-byte, fully used loads.
//
// Work decomposition (one workgroup per (sequence, KV head, context
// partition): 2 wave64s in the matrix-core kernel when the shape's full grid
// has 1024 or more workgroups, 4 otherwise and in the other kernels):
//   * a partition covers part_tokens consecutive positions; its 16-position
//     chunks are dealt round-robin to the waves; all G query heads of the KV
//     head share every K/V load;
//   * inside a wave, lanes are split into "rows"; each row is an independent
//     online-softmax stream over a fixed subset of the positions, so no
//     cross-row communication happens in the main loop;
//   * at the end the streams are merged with the log-sum-exp identity
//     (shuffles across rows, LDS across waves). A sequence with a single
//     partition writes its output directly; otherwise the partition's
//     (max, exp-sum, normalised output) go to the workspace and a second
//     kernel merges the partitions.
// Scores are kept in log2 units: q.k * scale * log2(e), exponentiated with
// v_exp_f32 (2^x).
//
// Two partition kernels:
//   VALU: 16-byte lane loads of K rows, per-lane partial dot products
//         reduced across the row's lanes with DPP; P.V on the VALU.
//   MFMA: q.K on the matrix cores (v_mfma_f32_16x16x32_bf16) with K as the
//         A operand and the group's query rows, replicated over the 16
//         columns, as B; the result leaves each lane with the scores of its
//         own row's 4 positions. P.V on the matrix cores too
//         (v_mfma_f32_16x16x16_bf16, each lane's own V rows and weights as
//         operands) for 2+ query heads per KV head and 8-bit pools; at one
//         head, a quad-level DPP broadcast of the probabilities and P.V on
//         the VALU.
// Every device-resident index is range-checked; a bad one is replaced by an
// in-range value, its work is masked, and a bit is set in g_error_word.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "pa_internal.h"

namespace pa {

__device__ uint32_t g_error_word;

namespace {

constexpr uint32_t kErrBlockId = 0x1u;
constexpr uint32_t kErrSeqLen = 0x2u;
constexpr uint32_t kErrSlot = 0x4u;
constexpr uint32_t kErrCopyPair = 0x8u;
constexpr uint32_t kErrQuery = 0x10u;
constexpr uint32_t kErrPrefix = 0x20u;
constexpr uint32_t kErrPlan = 0x40u;

__device__ __forceinline__ void flag_error(uint32_t bit) { atomicOr(&g_error_word, bit); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerLoad = 4;
  __device__ static __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ void store(float* p, float x) { *p = x; }
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPerLoad = 8;
  __device__ static __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = lo_bf16(v.x);
    f[1] = hi_bf16(v.x);
    f[2] = lo_bf16(v.y);
    f[3] = hi_bf16(v.y);
    f[4] = lo_bf16(v.z);
    f[5] = hi_bf16(v.z);
    f[6] = lo_bf16(v.w);
    f[7] = hi_bf16(v.w);
  }
  __device__ static __forceinline__ void store(uint16_t* p, float x) { *p = to_bf16(x); }
};

// Four consecutive outputs (16-byte aligned for fp32, 8-byte for bf16).
template <typename T>
__device__ __forceinline__ void store4(T* p, float x0, float x1, float x2, float x3);
template <>
__device__ __forceinline__ void store4<float>(float* p, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float x0, float x1, float x2,
                                                 float x3) {
  const uint32_t lo = (uint32_t)to_bf16(x0) | ((uint32_t)to_bf16(x1) << 16);
  const uint32_t hi = (uint32_t)to_bf16(x2) | ((uint32_t)to_bf16(x3) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

// N consecutive elements (N = 1 or 2, aligned to N elements) as floats.
template <typename T, int N>
__device__ __forceinline__ void load_elems(const T* p, float (&f)[N]) {
  static_assert(N == 1 || N == 2, "one or two elements");
  if constexpr (std::is_same<T, float>::value) {
    if constexpr (N == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      f[0] = v.x;
      f[1] = v.y;
    } else {
      f[0] = *p;
    }
  } else {
    if constexpr (N == 2) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
      f[0] = lo_bf16(v);
      f[1] = hi_bf16(v);
    } else {
      f[0] = __uint_as_float((uint32_t)*p << 16);
    }
  }
}

__device__ __forceinline__ uint4 ld16(const char* base, uint32_t byte_off) {
  return *reinterpret_cast<const uint4*>(base + byte_off);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each group of LPR consecutive lanes (LPR in 8, 16, 32); every
// lane of the group receives the total.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "lanes per row");
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: lane k <- 7-k within 8
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror: lane k <- 15-k
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Value held by lane (k & ~(G-1)) + h of this lane's quad, for every lane k.
template <int G, int H>
__device__ __forceinline__ float quad_pick(float x) {
  static_assert(G == 1 || G == 2 || G == 4, "quad group");
  if constexpr (G == 1) {
    return x;
  } else {
    constexpr int s0 = (0 & ~(G - 1)) | H, s1 = (1 & ~(G - 1)) | H;
    constexpr int s2 = (2 & ~(G - 1)) | H, s3 = (3 & ~(G - 1)) | H;
    return dpp<s0 | (s1 << 2) | (s2 << 4) | (s3 << 6)>(x);
  }
}

// out[h] = the value held by the lane of this quad that owns head h.
template <int G>
__device__ __forceinline__ void quad_spread(float x, float (&out)[G]) {
  if constexpr (G == 1) {
    out[0] = x;
  } else if constexpr (G == 2) {
    out[0] = quad_pick<2, 0>(x);
    out[1] = quad_pick<2, 1>(x);
  } else {
    out[0] = quad_pick<4, 0>(x);
    out[1] = quad_pick<4, 1>(x);
    out[2] = quad_pick<4, 2>(x);
    out[3] = quad_pick<4, 3>(x);
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Online softmax with a lazy reference maximum: a stream's reference m (log2
// units) moves only when a new score exceeds it by more than kLazyMax, so
// after its first positions a stream almost never rescales its output, and
// each exponent exp2(s - m) stays at most 2^kLazyMax. The result is the same
// softmax for any reference (m only scales the terms and the sum alike).
constexpr float kLazyMax = 8.0f;

// max(a, b, c) in one v_max3_f32. For matrix-core results the compiler
// otherwise quiets each operand with a max of the value with itself before
// every two-input max (it cannot tell they hold no signalling NaN).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max(a, |b|, |c|) in one v_max3_f32 with absolute-value operand modifiers
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Two bf16 halves of 32-bit words into one word: the low halves of lo_src
// (bits 0-15) and hi_src (bits 16-31), or their high halves, in one v_perm_b32.
__device__ __forceinline__ uint32_t pack_low_halves(uint32_t lo_src, uint32_t hi_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_high_halves(uint32_t lo_src, uint32_t hi_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);
}

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// Two floats as a bf16 pair (round to nearest even), low element first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2v_t __attribute__((ext_vector_type(2)));
  const f32x2v_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v_t));
}

// Two floats as an fp16 pair (round to nearest even), low element first.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef float f32x2v_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));
  const f32x2v_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2v_t));
}

// Weight of a softmax stream with running max m when merged under max M.
__device__ __forceinline__ float merge_weight(float m, float big_m) {
  return m == -INFINITY ? 0.0f : exp2_fast(m - big_m);
}

// Validated view of one sequence / partition for a workgroup.
struct PartitionWork {
  int i, g, j;       // sequence, KV head, partition
  int len;           // validated sequence length
  int nparts;        // partitions of this sequence
  int tok0, tok1;    // positions [tok0, tok1) of partition j
  int slot;          // partial slot of partition j
  bool direct;       // the partition is the whole walk: write out itself
};

// Start of sequence i's walk for shared-prefix decode (0 otherwise); an
// invalid start is flagged and replaced by 0 (the reduce does the same).
__device__ __forceinline__ int walk_start(const DecodeArgs& a, int i, int len, bool flag) {
  if (!a.pos_start) return 0;
  const int s = a.pos_start[i];
  if (s < 0 || s > len || s > a.max_prefix || s % a.block_size != 0) {
    if (flag) flag_error(kErrPrefix);
    return 0;
  }
  return s;
}

// Sequence length checked against the host bound (len_cap = min(max_seq_len,
// max_blocks * bs)); out-of-range values are clamped and flagged.
__device__ __forceinline__ int checked_len(const DecodeArgs& a, int i) {
  int len = a.seq_lens[i];
  if (len < 0 || len > a.len_cap) {
    if (threadIdx.x == 0) flag_error(kErrSeqLen);
    len = len < 0 ? 0 : a.len_cap;
  }
  return len;
}

__device__ __forceinline__ int checked_block(const DecodeArgs& a, int i, int logical_block) {
  int b = a.block_tables[(int64_t)i * a.max_blocks + logical_block];
  b = __builtin_amdgcn_readfirstlane(b);
  if ((unsigned)b >= (unsigned)a.num_blocks) {
    if ((threadIdx.x & 63) == 0) flag_error(kErrBlockId);
    b = 0;
  }
  return b;
}

// Writes zeros for the G query heads of KV head g of a sequence with no
// cached tokens.
template <typename T, int D, int G, int NW>
__device__ void write_zero_rows(const DecodeArgs& a, int i, int g) {
  T* out = reinterpret_cast<T*>(a.out);
  for (int t = threadIdx.x; t < G * D; t += NW * 64) {
    const int h = t / D, d = t % D;
    Elem<T>::store(out + ((int64_t)i * a.num_q_heads + g * G + h) * D + d, 0.0f);
  }
}

// Merges the NW waves' streams staged in LDS (s_m[w][h], s_l[w][h]: each
// wave's (max, exp-sum) per head, s_acc[w][h][d]: its unnormalised output)
// and writes either the final output (single-partition sequence) or the
// partition's partials. Called by every thread after the staging barrier.
template <typename T, int D, int G, int NW, bool PFX>
__device__ __forceinline__ void finish_waves(const DecodeArgs& a, const PartitionWork& wk,
                                             const float (*s_m)[G], const float (*s_l)[G],
                                             const float (*s_acc)[G][D], float out_scale) {
  // Merge of the NW wave streams, 4 consecutive dims per thread: one 16-byte
  // (fp32) or 8-byte (bf16) store each.
  constexpr int V4 = D / 4;
  for (int t = threadIdx.x; t < G * V4; t += NW * 64) {
    const int h = t / V4, d0 = (t % V4) * 4;
    float big = -INFINITY;
#pragma unroll
    for (int k = 0; k < NW; ++k) big = fmaxf(big, s_m[k][h]);
    float lsum = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float f = merge_weight(s_m[k][h], big);
      lsum += f * s_l[k][h];
      const float4 sa = *reinterpret_cast<const float4*>(&s_acc[k][h][d0]);
      o[0] += f * sa.x;
      o[1] += f * sa.y;
      o[2] += f * sa.z;
      o[3] += f * sa.w;
    }
    const float inv = lsum > 0.0f ? out_scale / lsum : 0.0f;
    const int64_t row = (int64_t)wk.i * a.num_q_heads + wk.g * G + h;
    if (wk.direct) {
      store4<T>(reinterpret_cast<T*>(a.out) + row * D + d0, o[0] * inv, o[1] * inv, o[2] * inv,
                o[3] * inv);
    } else {
      // the partial output of a partition holding at least
      // kHalfPartialMinTokens positions is stored in bf16 when part_half is
      // set (in the first half of its fp32-sized slot), other partials in
      // fp32; the merge of the partitions runs in fp32
      float* slot = reinterpret_cast<float*>(a.part_o) +
                    (row * (PFX ? a.slot_stride : a.max_parts) + wk.slot) * D;
      if (a.part_half && wk.tok1 - wk.tok0 >= kHalfPartialMinTokens)
        store4<uint16_t>(reinterpret_cast<uint16_t*>(slot) + d0, o[0] * inv, o[1] * inv,
                         o[2] * inv, o[3] * inv);
      else
        store4<float>(slot + d0, o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
  }
  // (max, exp-sum) of every head of the group: one full 128-byte record per
  // workgroup, so the write never covers part of a cache line.
  if (!wk.direct && threadIdx.x < kMlRecord / 4) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int f = threadIdx.x * 4 + e, h = f >> 1;
      v[e] = 0.0f;
      if (h < G) {
        float big = -INFINITY;
#pragma unroll
        for (int k = 0; k < NW; ++k) big = fmaxf(big, s_m[k][h]);
        float lsum = 0.0f;
#pragma unroll
        for (int k = 0; k < NW; ++k) lsum += merge_weight(s_m[k][h], big) * s_l[k][h];
        v[e] = (f & 1) ? lsum : big;
      }
    }
    const int64_t rec = (((int64_t)wk.i * a.num_kv_heads + wk.g) *
                             (PFX ? a.slot_stride : a.max_parts) + wk.slot) * kMlRecord;
    reinterpret_cast<float4*>(a.part_ml + rec)[threadIdx.x] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Merges the per-row softmax streams of every wave and writes either the
// final output (single-partition sequence) or the partition's partials.
// Inputs per lane: m[h], l[h] of the lane's row stream (log2 units) and
// acc[h][e] = unnormalised output for dims c*EPL + e, where c = lane % LPR.
#ifndef PA_FINISH_PERMLANE
#define PA_FINISH_PERMLANE 1
#endif

// Value held by lane (lane ^ OFF), for OFF in {16, 32}: the permlane swap
// instructions exchange 16- or 32-lane halves between two registers on the
// VALU, with no trip through LDS.
template <int OFF>
__device__ __forceinline__ float xor_lanes(float x) {
  static_assert(OFF == 16 || OFF == 32, "row exchange");
  const uint32_t u = __float_as_uint(x);
  const int lane = threadIdx.x & 63;
  if constexpr (OFF == 32) {
    // first: lanes 32-63 take lanes 0-31 of the second operand;
    // second: lanes 0-31 take lanes 32-63 of the first operand
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
  } else {
    // same exchange between odd and even 16-lane rows
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  }
}

template <int OFF>
__device__ __forceinline__ float row_partner(float x) {
#if PA_FINISH_PERMLANE
  if constexpr (OFF == 16 || OFF == 32) return xor_lanes<OFF>(x);
#endif
  return __shfl_xor(x, OFF);
}

// Merges the per-row softmax streams of every wave and writes either the
// final output (single-partition sequence) or the partition's partials.
// Inputs per lane: m[h], l[h] of the lane's row stream (log2 units) and
// acc[h][e] = unnormalised output for dims c*EPL + e, where c = lane % LPR.
template <typename T, int D, int G, int NW, int LPR, int EPL, bool PFX = false>
__device__ __forceinline__ void finish_partition(const DecodeArgs& a, const PartitionWork& wk,
                                                 float (&m)[G], float (&l)[G],
                                                 float (&acc)[G][EPL], float out_scale = 1.0f) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane % LPR;
  // rows of one wave: butterfly over the lane bits above the row
  auto merge_rows = [&](auto off_tag) {
    constexpr int OFF = decltype(off_tag)::value;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = row_partner<OFF>(m[h]);
      const float lo = row_partner<OFF>(l[h]);
      const float big = fmaxf(m[h], mo);
      const float f1 = merge_weight(m[h], big), f2 = merge_weight(mo, big);
      l[h] = f1 * l[h] + f2 * lo;
      m[h] = big;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = row_partner<OFF>(acc[h][e]);
        acc[h][e] = f1 * acc[h][e] + f2 * ao;
      }
    }
  };
  if constexpr (LPR <= 8) merge_rows(std::integral_constant<int, 8>{});
  if constexpr (LPR <= 16) merge_rows(std::integral_constant<int, 16>{});
  if constexpr (LPR <= 32) merge_rows(std::integral_constant<int, 32>{});
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ __align__(16) float s_acc[NW][G][D];
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[w][h][c * EPL + e] = acc[h][e];
      if (c == 0) {
        s_m[w][h] = m[h];
        s_l[w][h] = l[h];
      }
    }
  }
  __syncthreads();
  finish_waves<T, D, G, NW, PFX>(a, wk, s_m, s_l, s_acc, out_scale);
}


// Work units are (sequence i, KV head g, partition j), one per workgroup.
// Workgroup ids are dealt to the 8 XCDs round-robin (XCD x = id % 8). When
// Hkv is a multiple of 8, round r = id / 8 names (sequence i, block of 8 KV
// heads, partition j), partition fastest, and XCD x takes KV head
// g = 8 * block + (x - j) mod 8: each round hands every XCD a unit of the
// same (i, j), so the XCDs get equal work whatever the lengths, and a given
// (g, j) always lands on XCD (g + j) mod 8, so sequences sharing prompt
// blocks meet in one L2. Otherwise units are numbered partition fastest,
// then head, then sequence.
// Decodes workgroup id `id`; returns false if the workgroup has nothing to do
// (after writing zeros for an empty sequence).
// With a work plan (a.plan), unit u = (sequence, partition, length) comes
// from a.plan[u] instead: rounds name (unit, block of 8 KV heads), head block
// fastest, the same XCD deal inside a round; without Hkv % 8 == 0, KV head
// fastest, then unit. The grid then holds only units with work, in the
// plan's order.
template <typename T, int D, int BS, int G, int NW, bool PFX = false>
__device__ __forceinline__ bool setup_partition(const DecodeArgs& a, PartitionWork& wk,
                                                int id) {
  if (a.plan) {
    // entry (sequence, partition, sequence length, walk start): the length
    // comes with the unit, so no dependent load of seq_lens precedes the
    // table window (the start of a shared-prefix walk is read from
    // pos_start, as without a plan)
    int4 e;
    if (a.num_kv_heads % 8 == 0) {
      const int x = id & 7, r = id >> 3, nb8 = a.num_kv_heads >> 3;
      e = reinterpret_cast<const int4*>(a.plan)[r / nb8];
      wk.g = (r % nb8) * 8 + ((x - e.y) & 7);
    } else {
      e = reinterpret_cast<const int4*>(a.plan)[id / a.num_kv_heads];
      wk.g = id % a.num_kv_heads;
    }
    wk.i = e.x;
    wk.j = e.y;
    wk.len = e.z;
    bool bad = (unsigned)wk.i >= (unsigned)a.num_seqs || (unsigned)wk.len > (unsigned)a.len_cap ||
               wk.j < 0;
    if (!bad) {
      const int st = PFX && wk.len > 0 ? walk_start(a, wk.i, wk.len, false) : 0;
      const int np = (wk.len - st + a.part_tokens - 1) / a.part_tokens;
      bad = wk.j >= (np > 1 ? np : 1);
    }
    if (bad) {
      if (threadIdx.x == 0) flag_error(kErrPlan);
      return false;
    }
  } else if (a.num_kv_heads % 8 == 0) {
    const int x = id & 7, r = id >> 3;
    wk.j = r % a.max_parts;
    const int rest = r / a.max_parts, nb8 = a.num_kv_heads >> 3;
    wk.g = (rest % nb8) * 8 + ((x - wk.j) & 7);
    wk.i = rest / nb8;
  } else {
    wk.j = id % a.max_parts;
    const int rest = id / a.max_parts;
    wk.g = rest % a.num_kv_heads;
    wk.i = rest / a.num_kv_heads;
  }
  if (!a.plan) wk.len = checked_len(a, wk.i);
  if (wk.len == 0) {
    if (wk.j == 0) write_zero_rows<T, D, G, NW>(a, wk.i, wk.g);
    return false;
  }
  // PFX: shared-prefix decode's per-sequence walk (starts after the prefix,
  // always leaves partials, in slots from slot0)
  const int start = PFX ? walk_start(a, wk.i, wk.len, threadIdx.x == 0) : 0;
  wk.nparts = (wk.len - start + a.part_tokens - 1) / a.part_tokens;
  if (wk.j >= wk.nparts) return false;
  wk.tok0 = start + wk.j * a.part_tokens;
  wk.tok1 = min(wk.len, wk.tok0 + a.part_tokens);
  wk.slot = PFX ? a.slot0 + wk.j : wk.j;
  wk.direct = !PFX && wk.nparts == 1;
  return true;
}

// ---------------------------------------------------------------------------
// VALU partition kernel
// ---------------------------------------------------------------------------
template <typename T, int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partition_valu(DecodeArgs a) {
  constexpr int S = sizeof(T);
  constexpr int EPL = Elem<T>::kPerLoad;  // elements per 16-byte lane load
  constexpr int LPR = D / EPL;            // lanes holding one token row
  constexpr int RPI = 64 / LPR;           // token rows per wave-wide load
  constexpr int NLB = BS / RPI;           // loads per block per lane
  static_assert(LPR * 16 == D * S, "row must split into 16-byte lane chunks");
  constexpr int64_t kHeadBytes = (int64_t)BS * D * S;

  PartitionWork wk;
  if (!setup_partition<T, D, BS, G, NW>(a, wk, blockIdx.x)) return;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR, c = lane % LPR;
  const int64_t blk_bytes = kHeadBytes * a.num_kv_heads;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + wk.g * kHeadBytes;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + wk.g * kHeadBytes;

  float qf[G][EPL];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((int64_t)wk.i * a.num_q_heads + wk.g * G) * D + c * EPL) * S;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      Elem<T>::unpack(ld16(qp, h * D * S), qf[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] *= a.qscale;
    }
  }
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }

  const int blk0 = wk.tok0 / BS;
  const int nblk = (wk.tok1 - wk.tok0 + BS - 1) / BS;
  for (int b = w; b < nblk; b += NW) {
    const int lb = blk0 + b;
    const int phys = checked_block(a, wk.i, lb);
    const char* kb = kbase + (int64_t)phys * blk_bytes;
    const char* vb = vbase + (int64_t)phys * blk_bytes;
    uint4 kr[NLB], vr[NLB];
#pragma unroll
    for (int n = 0; n < NLB; ++n) kr[n] = ld16(kb, n * RPI * D * S + lane * 16);
#pragma unroll
    for (int n = 0; n < NLB; ++n) vr[n] = ld16(vb, n * RPI * D * S + lane * 16);

    const int pos0 = lb * BS + r;  // position of this row's first token
    const bool full = lb * BS + BS <= wk.tok1;
    float s[NLB][G];
#pragma unroll
    for (int n = 0; n < NLB; ++n) {
      float kf[EPL];
      Elem<T>::unpack(kr[n], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) t = fmaf(qf[h][e], kf[e], t);
        s[n][h] = group_sum<LPR>(t);
      }
    }
    bool ok[NLB];
#pragma unroll
    for (int n = 0; n < NLB; ++n) ok[n] = full || (pos0 + n * RPI < wk.tok1);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = -INFINITY;
#pragma unroll
      for (int n = 0; n < NLB; ++n) bm = ok[n] ? fmaxf(bm, s[n][h]) : bm;
      const float mn = fmaxf(m[h], bm);
      const float alpha = mn == m[h] ? 1.0f : exp2_fast(m[h] - mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int n = 0; n < NLB; ++n) {
      float vf[EPL];
      Elem<T>::unpack(vr[n], vf);
      if (!full) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = ok[n] ? vf[e] : 0.0f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = ok[n] ? exp2_fast(s[n][h] - m[h]) : 0.0f;
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  }
  finish_partition<T, D, G, NW, LPR, EPL>(a, wk, m, l, acc);
}

// ---------------------------------------------------------------------------
// MFMA partition kernel (bf16 or 8-bit pools, D = 128, G in {1, 2, 4})
// ---------------------------------------------------------------------------
// Positions are taken 16 at a time ("chunk"; a 16-token block, or a 16-token
// slice of a larger block). Lane l: R = l / 16 (row), c = l % 16.
//   K load s (s = 0..3): token (l % 16), dims [32 s + 8 R, +8)  -> A operand
//   q operand step s:    query row (l % 16) % G, same dims        -> B operand
//   MFMA result reg r:   score of token 4 R + r for head (l % G)
//   V load jj (0..3):    token 4 R + jj, dims [8 c, +8), coalesced 256 B rows
// With P.V on the VALU (one query head per KV head) row R is one softmax
// stream over tokens {4R .. 4R+3} of every chunk; with P.V on the matrix
// cores the four rows share one stream per head (mfma_chunk_pvm).
//
// Wave w of the workgroup takes chunks w, w + NW, w + 2 NW, ... of the
// partition. The physical block ids of those chunks are read once, one per
// lane, into a register window of 64 chunks (re-read only for partitions of
// more than 64 * NW chunks), and broadcast per chunk with a lane read, so the
// K/V loads never wait for a block-table load. K/V of the next chunk are
// issued before the current chunk is computed (two register buffers); the
// last chunk "prefetches" itself again, a cache hit that keeps the load
// count per iteration constant.
// One 16-token chunk of K and V rows in registers, with the operand views
// the matrix-core kernel needs: kop(s) = the bf16x8 A operand of q.K step s,
// vrow(jj, f) = the 8 V values of the lane's jj-th row as floats.
struct KVChunk {                       // bf16 pools
  uint4 k[4];
  uint4 v[4];
  __device__ __forceinline__ bf16x8_t kop(int s) const { return __builtin_bit_cast(bf16x8_t, k[s]); }
  __device__ __forceinline__ void vrow(int jj, float (&f)[8]) const {
    Elem<uint16_t>::unpack(v[jj], f);
  }
};

// Two FP8 E4M3 codes (bytes 0-1, or 2-3 with HI) of a word as a bf16 pair.
// The hardware conversion is exact (an E4M3 value has 4 significant bits),
// so is dropping the float's low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two E4M3 codes (bytes 0-1, or 2-3 with HI) to two bf16: one gfx950
// v_cvt_scalef32_pk_bf16_fp8 at scale 1.0. Exact: every E4M3 value,
// subnormals included, is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  const bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

template <bool HI>
__device__ __forceinline__ void e4m3x2_to_f32(uint32_t w, float& a, float& b) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  a = f[0];
  b = f[1];
}

struct KVChunk8 {                      // FP8 E4M3 pools: 128-byte rows
  uint4 k[2];                          // dims 16R + 64 h .. +16 for h = 0, 1
  uint2 v[4];                          // dims 8c .. 8c + 7 of rows 4R + jj
  __device__ __forceinline__ bf16x8_t kop(int s) const {
    const uint4& w = k[s >> 1];
    const uint32_t lo = (s & 1) ? w.z : w.x, hi = (s & 1) ? w.w : w.y;
    const uint4 r = make_uint4(e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo),
                               e4m3x2_to_bf16x2<false>(hi), e4m3x2_to_bf16x2<true>(hi));
    return __builtin_bit_cast(bf16x8_t, r);
  }
  __device__ __forceinline__ void vrow(int jj, float (&f)[8]) const {
    e4m3x2_to_f32<false>(v[jj].x, f[0], f[1]);
    e4m3x2_to_f32<true>(v[jj].x, f[2], f[3]);
    e4m3x2_to_f32<false>(v[jj].y, f[4], f[5]);
    e4m3x2_to_f32<true>(v[jj].y, f[6], f[7]);
  }
};

// Occupancy floor of the MFMA partition kernel (waves per SIMD; 0 = the
// compiler's choice) and the cache-policy bits of its K/V loads.
#ifndef PA_MFMA_WAVES_PER_EU
#define PA_MFMA_WAVES_PER_EU 0
#endif
#if PA_MFMA_WAVES_PER_EU > 0
#define PA_MFMA_BOUNDS(threads) __launch_bounds__(threads, PA_MFMA_WAVES_PER_EU)
#else
#define PA_MFMA_BOUNDS(threads) __launch_bounds__(threads)
#endif
// Cache policies of the K/V loads (the buffer instructions' cache-policy
// operand). Streaming (nt, non-temporal) is the default: each V line is
// read once, and on the Llama-3-8B-shaped decode it takes about 4% off the
// partition kernel. K lines are read in two halves by consecutive loads;
// with 2 or 4 query heads per KV head they keep the plain policy
// (mfma_unit). When sequences of one batch share blocks (forked samples, a
// common prompt), a sequence reads lines that its neighbours in the grid
// just brought into L2; the plain policy keeps them there.
constexpr int kKvStream = 2;
constexpr int kKvCached = 0;
// depth of the K/V register pipeline of the matrix-core partition kernel
#ifndef PA_PIPE_BF16
#define PA_PIPE_BF16 2
#endif
#ifndef PA_PIPE_F8
#define PA_PIPE_F8 2
#endif

// Buffer resource over `bytes` bytes at a wave-uniform address (gfx9
// descriptor: raw 32-bit data format, no swizzle); loads past `bytes` return
// zeros instead of touching memory (so a descriptor of 0 bytes makes a load
// that only keeps the wait counts regular).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, 0x00020000);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes at voff + soff of the buffer (soff wave-uniform), cache policy POL.
template <int POL>
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL);
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int POL>
__device__ __forceinline__ uint2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POL);
  return make_uint2(v.x, v.y);
}

// FP8 pools: K rows as two 16-byte loads per lane (dims 16R + 64h), V rows
// as four 8-byte loads (dims 8c of rows 4R + jj); 2 KiB per chunk and pool.
template <int BS, int POL = kKvStream, int KPOL = POL>
__device__ __forceinline__ void load_kv_chunk(KVChunk8& c, const char* kbase, const char* vbase,
                                              int64_t blk_bytes, int phys, int tok_in_blk,
                                              uint32_t k_off, uint32_t v_off, bool live) {
  constexpr int ROW = 128;
  const int64_t base = (int64_t)phys * blk_bytes + (int64_t)tok_in_blk * ROW;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + base, live ? 16 * ROW : 0);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + base, live ? 16 * ROW : 0);
  c.k[0] = buf_ld16<KPOL>(kr, k_off, 0);    // the two halves of each K line
  c.k[1] = buf_ld16<KPOL>(kr, k_off, 64);   // (see the 16-bit form below)
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) c.v[jj] = buf_ld8<POL>(vr, v_off, jj * ROW);
}

// K and V rows of the 16-token chunk that starts at row `tok_in_blk` of
// physical block `phys`. The chunk's base address is wave-uniform and goes
// into the buffer descriptor (scalar registers); each lane only adds its own
// fixed offset, so no per-lane 64-bit address is formed per chunk.
template <int BS, int POL = kKvStream, int KPOL = POL>
__device__ __forceinline__ void load_kv_chunk(KVChunk& c, const char* kbase, const char* vbase,
                                              int64_t blk_bytes, int phys, int tok_in_blk,
                                              uint32_t k_off, uint32_t v_off, bool live) {
  constexpr int ROW = 256;
  const int64_t base = (int64_t)phys * blk_bytes + (int64_t)tok_in_blk * ROW;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + base, live ? 16 * ROW : 0);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + base, live ? 16 * ROW : 0);
  // K: one load covers 64 bytes of each of 16 token rows, so loads s and
  // s + 1 read the two halves of the same 128-byte lines; with the plain
  // policy (KPOL) the second half is an L1 hit, where streaming K loads
  // fetch each line twice from L2. V loads cover whole rows and keep POL.
#pragma unroll
  for (int s = 0; s < 4; ++s) c.k[s] = buf_ld16<KPOL>(kr, k_off, s * 64);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) c.v[jj] = buf_ld16<POL>(vr, v_off, jj * ROW);
}

// 16-token chunk that spans two 8-token blocks: lanes pick their block per
// row, so the loads use per-lane 64-bit addresses instead of a descriptor.
__device__ __forceinline__ void load_kv_chunk_bs8(KVChunk& c, const char* kbase, const char* vbase,
                                                  int64_t blk_bytes, int phys0, int phys1) {
  constexpr int ROW = 256;
  const int lane = threadIdx.x & 63, R = lane >> 4, cc = lane & 15;
  // K: token cc of the chunk; V: tokens 4R .. 4R + 3
  const char* kb = kbase + (int64_t)(cc < 8 ? phys0 : phys1) * blk_bytes + (cc & 7) * ROW + R * 16;
  const char* vb = vbase + (int64_t)(R < 2 ? phys0 : phys1) * blk_bytes + ((4 * R) & 7) * ROW +
                   cc * 16;
#pragma unroll
  for (int s = 0; s < 4; ++s) c.k[s] = ld16(kb, s * 64);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) c.v[jj] = ld16(vb, jj * ROW);
}

__device__ __forceinline__ int checked_id(const int32_t* tables, int32_t num_blocks, int64_t row,
                                          int logical_block) {
  int id = tables[row + logical_block];
  if ((unsigned)id >= (unsigned)num_blocks) {
    flag_error(kErrBlockId);
    id = 0;
  }
  return id;
}

// Block-id window: lane k gets the physical block holding the start of this
// wave's chunk (first + k), for chunks inside the partition; other lanes get
// 0. With 8-token blocks a chunk covers two blocks; .y is the second one
// (read only when the chunk has a valid position in it). Each id is
// range-checked here, once.
template <int BS, int NW>
__device__ __forceinline__ int2 load_id_window(const DecodeArgs& a, const PartitionWork& wk, int w,
                                               int first, int nmine) {
  const int lane = threadIdx.x & 63;
  const int k = first + lane;
  int2 id = make_int2(0, 0);
  if (k < nmine) {
    const int tok = wk.tok0 + (w + k * NW) * 16;
    const int64_t row = (int64_t)wk.i * a.max_blocks;
    id.x = checked_id(a.block_tables, a.num_blocks, row, tok / BS);
    id.y = id.x;
    if constexpr (BS == 8) {
      if (tok + 8 < wk.tok1) id.y = checked_id(a.block_tables, a.num_blocks, row, tok / 8 + 1);
    }
  }
  return id;
}

template <int G, typename CH>
__device__ __forceinline__ void mfma_chunk(const CH& c, const bf16x8_t (&qop)[4],
                                           float qscale, int tokc, int tok1, int R, float& m,
                                           float& lsum, float (&acc)[G][8]) {
  f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.kop(s), qop[s], sc, 0, 0, 0);
  const bool full = tokc + 16 <= tok1;
  float sv[4];
  bool ok[4];
  float bm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sv[r] = sc[r] * qscale;
    ok[r] = full || (tokc + 4 * R + r < tok1);
    bm = ok[r] ? fmaxf(bm, sv[r]) : bm;
  }
  const float mn = bm > m + kLazyMax ? bm : m;
  const float alpha = mn == m ? 1.0f : exp2_fast(m - mn);
  m = mn;
  float p[4];
  float psum = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = ok[r] ? exp2_fast(sv[r] - mn) : 0.0f;
    psum += p[r];
  }
  lsum = lsum * alpha + psum;
  float ph[4][G];
#pragma unroll
  for (int r = 0; r < 4; ++r) quad_spread<G>(p[r], ph[r]);
  // rescale only when some stream of the wave moved its reference
  if (__ballot(alpha != 1.0f) != 0) {
    float al[G];
    quad_spread<G>(alpha, al);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float vf[8];
    c.vrow(jj, vf);
    if (!full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] = ok[jj] ? vf[e] : 0.0f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph[jj][h], vf[e], acc[h][e]);
  }
}

// P.V on the matrix cores too (v_mfma_f32_16x16x16_bf16), each lane feeding
// its own values (used for 8-bit pools and for 2+ query heads per KV head). A = V^T for dims 8m + t (tile t = 0..7, row m
// = lane % 16): lane (R, c) holds the codes of rows 4R .. 4R+3 at dims 8c ..
// 8c+7, i.e. exactly A[m = c][k = 4R .. 4R+3] of every tile (8-bit codes
// converted to bf16, exactly). B = P: lane (R, c) holds the weights of those rows
// for head c % G, B[k = 4R .. 4R+3][n = c], as two bf16 terms. The result
// C[m = 4R + r][n = c] of tile t is O[head c % G][dim 8 (4R + r) + t]. The
// four row groups feed one product, so each head is one softmax stream: the
// block maximum is shared across the row groups (two cross-lane steps) and
// every lane keeps its own share of the exp-sum.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

template <int G, typename CH>
__device__ __forceinline__ void mfma_chunk_pvm(const CH& c, const bf16x8_t (&qop)[4],
                                               float qscale, int tokc, int tok1, int R, float& m,
                                               float& lsum, f32x4_t (&acc)[8]) {
  f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.kop(s), qop[s], sc, 0, 0, 0);
  const bool full = tokc + 16 <= tok1;
  float sv[4];
  bool ok[4];
  float bm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sv[r] = sc[r] * qscale;
    ok[r] = full || (tokc + 4 * R + r < tok1);
    bm = ok[r] ? fmaxf(bm, sv[r]) : bm;
  }
  bm = fmaxf(bm, xor_lanes<16>(bm));
  bm = fmaxf(bm, xor_lanes<32>(bm));
  const float mn = bm > m + kLazyMax ? bm : m;
  const float alpha = mn == m ? 1.0f : exp2_fast(m - mn);
  m = mn;
  float p[4];
  float psum = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = ok[r] ? exp2_fast(sv[r] - mn) : 0.0f;
    psum += p[r];
  }
  lsum = lsum * alpha + psum;
  if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= alpha;
  }
  // B: the weights as two bf16 terms (hi + lo, ~16 significant bits)
  const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
  const uint32_t l01 = pack_bf16x2(p[0] - __uint_as_float(h01 << 16), p[1] - __uint_as_float(h01 & 0xffff0000u));
  const uint32_t l23 = pack_bf16x2(p[2] - __uint_as_float(h23 << 16), p[3] - __uint_as_float(h23 & 0xffff0000u));
  const bf16x4_t phi = __builtin_bit_cast(bf16x4_t, make_uint2(h01, h23));
  const bf16x4_t plo = __builtin_bit_cast(bf16x4_t, make_uint2(l01, l23));
  // A: bf16 pairs b[jj][u] = dims 8c + 2u, 8c + 2u + 1 of row 4R + jj (code
  // 0 for rows past the end, whose slack may hold NaN codes)
  uint32_t b[4][4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    if constexpr (std::is_same<CH, KVChunk8>::value) {
      const uint2 w = full || ok[jj] ? c.v[jj] : make_uint2(0, 0);
      b[jj][0] = e4m3x2_to_bf16x2<false>(w.x);
      b[jj][1] = e4m3x2_to_bf16x2<true>(w.x);
      b[jj][2] = e4m3x2_to_bf16x2<false>(w.y);
      b[jj][3] = e4m3x2_to_bf16x2<true>(w.y);
    } else {
      const uint4 w = full || ok[jj] ? c.v[jj] : make_uint4(0, 0, 0, 0);
      b[jj][0] = w.x;
      b[jj][1] = w.y;
      b[jj][2] = w.z;
      b[jj][3] = w.w;
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int u = t >> 1;
    const uint2 av = (t & 1) ? make_uint2(pack_high_halves(b[0][u], b[1][u]), pack_high_halves(b[2][u], b[3][u]))
                             : make_uint2(pack_low_halves(b[0][u], b[1][u]), pack_low_halves(b[2][u], b[3][u]));
    const bf16x4_t a = __builtin_bit_cast(bf16x4_t, av);
    acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, acc[t], 0, 0, 0);
    acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, acc[t], 0, 0, 0);
  }
}

// The waves' streams of the matrix-core P.V (mfma_chunk_pvm) into LDS, then
// finish_waves. Lane (R, c), c < G, holds head c: its max, the exp-sum of all
// row groups (l_all) and dims 32R + 8r + t in acc[t][r].
template <typename T, int D, int G, int NW, bool PFX>
__device__ __forceinline__ void finish_partition_pvm(const DecodeArgs& a, const PartitionWork& wk,
                                                     float m, float l_all, const f32x4_t (&acc)[8],
                                                     float out_scale) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, R = lane >> 4, c = lane & 15;
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ __align__(16) float s_acc[NW][G][D];
  if (c < G) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* d = &s_acc[w][c][32 * R + 8 * r];
      *reinterpret_cast<float4*>(d) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
      *reinterpret_cast<float4*>(d + 4) = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
    }
    if (R == 0) {
      s_m[w][c] = m;
      s_l[w][c] = l_all;
    }
  }
  __syncthreads();
  finish_waves<T, D, G, NW, PFX>(a, wk, s_m, s_l, s_acc, out_scale);
}

// One work unit (sequence, KV head, partition) of the matrix-core kernel.
// F8: the pools hold FP8 E4M3 codes (q and out stay bf16); scores use
// qscale = scale * log2(e) * k_scale and outputs are multiplied by v_scale.
template <int BS, int G, int NW, bool F8, bool PFX, int POL = kKvStream>
__device__ __forceinline__ void mfma_unit(const DecodeArgs& a, const PartitionWork& wk) {
  constexpr int D = 128;
  constexpr int ROW = F8 ? D : D * 2;             // bytes per token row
  constexpr int64_t kHeadBytes = (int64_t)BS * ROW;
  static_assert(BS == 8 || BS % 16 == 0, "block must hold whole 16-token chunks, or half of one");
  static_assert(!F8 || BS != 8, "8-bit pools take blocks of 16 tokens or more");
  using Chunk = typename std::conditional<F8, KVChunk8, KVChunk>::type;
  // register buffers in the K/V pipeline (an 8-bit chunk takes half the registers)
  constexpr int NBUF = BS == 8 ? 2 : (F8 ? PA_PIPE_F8 : PA_PIPE_BF16);
  // K loads with the plain policy when a group shares them (G 2, 4): 410 vs
  // 419 us on the Llama-3-8B shape, 234-237 vs 237-238 us with 8-bit pools;
  // at G 1 streaming stays faster (555 vs 567 us on the Llama-2-13B shape)
  constexpr int KPOL = G == 1 ? POL : kKvCached;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = lane >> 4, c = lane & 15;
  const int64_t blk_bytes = kHeadBytes * a.num_kv_heads;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + wk.g * kHeadBytes;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + wk.g * kHeadBytes;

  bf16x8_t qop[4];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((int64_t)wk.i * a.num_q_heads + wk.g * G + (lane % G)) * D + 8 * R) * 2;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // q.K step s covers dims 8R + 32s (bf16 pools) or 16R + 64(s/2) +
      // 8(s%2) (8-bit pools: the dims of a lane's two 16-byte K loads)
      const uint32_t off = F8 ? (uint32_t)(16 * R + 64 * (s >> 1) + 8 * (s & 1)) * 2 - 16 * R
                              : (uint32_t)s * 64;
      qop[s] = __builtin_bit_cast(bf16x8_t, ld16(qp, off));
    }
  }
  const uint32_t k_off = (uint32_t)(c * ROW + R * 16);       // + s * 64 (bf16), + h * 64 (8-bit)
  const uint32_t v_off = (uint32_t)(4 * R * ROW + c * (F8 ? 8 : 16));   // + jj * ROW

  float m = -INFINITY, lsum = 0.0f;  // stream of row R (8-bit pools: of the head), head lane % G
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  // P.V on the matrix cores (mfma_chunk_pvm) for 8-bit pools and for 2 or
  // more query heads per KV head; at one head the vector form needs few
  // instructions and stays slightly faster (Llama-2-13B shape: 570 vs 572 us)
  constexpr bool kPvm = F8 || (G > 1 && BS != 8);
  f32x4_t accm[8];                   // kPvm: the matrix-core P.V tiles
#pragma unroll
  for (int t = 0; t < 8; ++t) accm[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int nch = (wk.tok1 - wk.tok0 + 15) / 16;
  const int nmine = nch > w ? (nch - w + NW - 1) / NW : 0;   // chunks of this wave
  auto chunk_tok = [&](int t) { return wk.tok0 + (w + t * NW) * 16; };
  // Windows of 64 chunks: one block-id load per window, then a pipeline of
  // NBUF register buffers over the window's chunks: chunk t + NBUF - 1 is
  // issued before chunk t is computed. No load inside the loop depends on
  // another load, so the compiler's wait counts stay partial; issues past
  // the window's last chunk use an empty descriptor (no memory access; with
  // 8-token blocks, which use per-lane addresses, the last chunk again).
  for (int win = 0; win < nmine; win += 64) {
    const int2 ids = load_id_window<BS, NW>(a, wk, w, win, nmine);
    const int cnt = min(64, nmine - win);
    auto issue = [&](Chunk& buf, int t) {
      const bool live = t < cnt;
      const int tt = live ? t : cnt - 1;
      const int phys = __builtin_amdgcn_readlane(ids.x, tt);
      if constexpr (BS == 8) {
        load_kv_chunk_bs8(buf, kbase, vbase, blk_bytes, phys, __builtin_amdgcn_readlane(ids.y, tt));
      } else {
        load_kv_chunk<BS, POL, KPOL>(buf, kbase, vbase, blk_bytes, phys,
                                     chunk_tok(win + tt) % BS, k_off, v_off, live);
      }
    };
    // one stage: issue chunk t + NBUF - 1 into `nxt`, compute chunk t from
    // `cur`; true once the window is done. (Written out per depth: a loop
    // over a buffer array costs the compiler ~30 more registers.)
    int t = 0;
    auto stage = [&](Chunk& nxt, const Chunk& cur) {
      issue(nxt, t + NBUF - 1);
      if constexpr (kPvm)
        mfma_chunk_pvm<G>(cur, qop, a.qscale, chunk_tok(win + t), wk.tok1, R, m, lsum, accm);
      else
        mfma_chunk<G>(cur, qop, a.qscale, chunk_tok(win + t), wk.tok1, R, m, lsum, acc);
      return ++t >= cnt;
    };
    Chunk b0, b1;
    issue(b0, 0);
    if constexpr (NBUF == 2) {
      for (;;) {
        if (stage(b1, b0) || stage(b0, b1)) break;
      }
    } else if constexpr (NBUF == 3) {
      Chunk b2;
      issue(b1, 1);
      for (;;) {
        if (stage(b2, b0) || stage(b0, b1) || stage(b1, b2)) break;
      }
    } else {
      static_assert(NBUF == 4, "pipeline depth 2, 3 or 4");
      Chunk b2, b3;
      issue(b1, 1);
      issue(b2, 2);
      for (;;) {
        if (stage(b3, b0) || stage(b0, b1) || stage(b1, b2) || stage(b2, b3)) break;
      }
    }
  }
  if constexpr (kPvm) {
    float l_all = lsum + xor_lanes<16>(lsum);
    l_all += xor_lanes<32>(l_all);
    finish_partition_pvm<uint16_t, D, G, NW, PFX>(a, wk, m, l_all, accm, F8 ? a.out_scale : 1.0f);
  } else {
    float mh[G], lh[G];
    quad_spread<G>(m, mh);
    quad_spread<G>(lsum, lh);
    finish_partition<uint16_t, D, G, NW, 16, 8, PFX>(a, wk, mh, lh, acc, 1.0f);
  }
}

template <int BS, int G, int NW, bool F8, bool PFX = false, int POL = kKvStream>
// at least 3 waves per SIMD for the matrix-core P.V forms (unbounded, the
// compiler gives them 172 registers, 2 waves) and the shared-prefix walks
__global__ PA_MFMA_BOUNDS(NW * 64)
__attribute__((amdgpu_waves_per_eu(PFX || F8 || (G > 1 && BS != 8) ? 3 : 1)))
void decode_partition_mfma(DecodeArgs a) {
  PartitionWork wk;
  if (!setup_partition<uint16_t, 128, BS, G, NW, PFX>(a, wk, blockIdx.x)) return;
  mfma_unit<BS, G, NW, F8, PFX, POL>(a, wk);
}

// ---------------------------------------------------------------------------
// Partition merge
// ---------------------------------------------------------------------------
// One wave per (sequence, query head); only sequences with more than one
// partition have anything to merge.
// Partitions merged with every load issued up front (the common case).
constexpr int kReduceFast = 16;

template <typename T, int D, bool PFX = false>
__global__ __launch_bounds__(kReduceWaves * 64) void decode_reduce(DecodeArgs a) {
  // one wave per (sequence, query head); kReduceWaves consecutive pairs per
  // workgroup
  const int pair = blockIdx.x * kReduceWaves + (threadIdx.x >> 6);
  if (pair >= a.num_seqs * a.num_q_heads) return;
  const int hq = pair % a.num_q_heads;
  const int i = pair / a.num_q_heads;
  int len = a.seq_lens[i];
  len = len < 0 ? 0 : min(len, a.len_cap);
  if (len == 0) return;
  // partials k = 0 .. np - 1 of the row: with shared-prefix decode first the
  // prefix pass's np_pref slots (fp32), then the walk's own partitions
  const int pt = a.part_tokens;
  const int start = PFX ? walk_start(a, i, len, false) : 0;
  const int np_pref = PFX ? (start + a.prefix_part_tokens - 1) / a.prefix_part_tokens : 0;
  const int np = np_pref + (len - start + pt - 1) / pt;
  if (!PFX && np <= 1) return;                   // written by the partition kernel
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t stride = PFX ? a.slot_stride : a.max_parts;
  auto slot_of = [&](int k) { return PFX && k >= np_pref ? a.slot0 + (k - np_pref) : k; };
  // record of slot s: ml[s * kMlRecord] = (max, exp-sum) of this head
  const float* ml = a.part_ml +
                    ((int64_t)i * a.num_kv_heads + hq / G) * stride * kMlRecord + 2 * (hq % G);
  const int lane = threadIdx.x & 63;
  // partial k (see finish_partition for its storage type)
  const float* po = reinterpret_cast<const float*>(a.part_o) +
                    ((int64_t)i * a.num_q_heads + hq) * stride * D;
  // The lane's slice of partial k in two steps, so that the loads of a
  // batch can all be issued before any is decoded: raw_part loads the raw
  // words (D 128: one 8-byte load at the lane's bf16 or fp32 position, the
  // bf16 case reading 4 bytes past its pair, still inside the slot; D 64:
  // one 4-byte fp32 or 2-byte bf16 load), decode_part turns them into
  // floats.
  auto half_of = [&](int k) {
    const int t0 = start + (k - np_pref) * pt;
    return (!PFX || k >= np_pref) && a.part_half &&
           min(len, t0 + pt) - t0 >= kHalfPartialMinTokens;
  };
  auto raw_part = [&](int k, bool half) {
    const char* slot = reinterpret_cast<const char*>(po + (int64_t)slot_of(k) * D);
    uint2 w = make_uint2(0u, 0u);
    if constexpr (D / 64 == 2) {
      w = *reinterpret_cast<const uint2*>(slot + (half ? 4 : 8) * lane);
    } else if (half) {
      w.x = *reinterpret_cast<const uint16_t*>(slot + 2 * lane);
    } else {
      w.x = *reinterpret_cast<const uint32_t*>(slot + 4 * lane);
    }
    return w;
  };
  auto decode_part = [&](uint2 w, bool half, float (&f)[D / 64]) {
    if constexpr (D / 64 == 2) {
      f[0] = half ? lo_bf16(w.x) : __uint_as_float(w.x);
      f[1] = half ? hi_bf16(w.x) : __uint_as_float(w.y);
    } else {
      f[0] = half ? lo_bf16(w.x) : __uint_as_float(w.x);
    }
  };
  auto load_part = [&](int k, float (&f)[D / 64]) {
    const bool half = half_of(k);
    decode_part(raw_part(k, half), half, f);
  };
  constexpr int DPL = D / 64;
  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.0f;
  float wsum;
  if (np <= kReduceFast) {
    // every load up front: lane j's statistics, then each partition's slice
    const float mj = lane < np ? ml[(int64_t)slot_of(lane) * kMlRecord] : -INFINITY;
    const float lj = lane < np ? ml[(int64_t)slot_of(lane) * kMlRecord + 1] : 0.0f;
    // every load first; partitions past np (a wave-uniform test) load
    // nothing and count as zeros
    uint2 raw[kReduceFast];
    bool hf[kReduceFast];
#pragma unroll
    for (int j = 0; j < kReduceFast; ++j) {
      hf[j] = half_of(j);
      raw[j] = make_uint2(0u, 0u);
      if (j < np) raw[j] = raw_part(j, hf[j]);
    }
    float v[kReduceFast][DPL];
#pragma unroll
    for (int j = 0; j < kReduceFast; ++j) decode_part(raw[j], hf[j], v[j]);
    float big = mj;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) big = fmaxf(big, __shfl_xor(big, off));
    const float wj = lj * merge_weight(mj, big);
    wsum = wj;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
#pragma unroll
    for (int j = 0; j < kReduceFast; ++j) {
      const float w = __shfl(wj, j);
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] = fmaf(w, v[j][k], o[k]);
    }
  } else {
    // lane j folds partitions j, j + 64, ... into one (max, exp-sum) pair
    float mj = -INFINITY, lj = 0.0f;
    for (int k = lane; k < np; k += 64) {
      const int64_t j = slot_of(k);
      const float m2 = ml[j * kMlRecord], l2 = ml[j * kMlRecord + 1];
      const float big = fmaxf(mj, m2);
      lj = lj * merge_weight(mj, big) + l2 * merge_weight(m2, big);
      mj = big;
    }
    float big = mj;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) big = fmaxf(big, __shfl_xor(big, off));
    wsum = lj * merge_weight(mj, big);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
    if constexpr (D == 128) {
      // the four 16-lane rows take every fourth partition, 8 dims per lane
      // (dims 8c .. 8c + 7), four partitions' loads in flight at a time; the
      // rows' sums are then combined with 16/32-lane swaps
      const int R = lane >> 4, c = lane & 15;
      float acc8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      for (int k0 = R; k0 < np; k0 += 16) {
        float wv[4], v[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = k0 + 4 * u < np ? k0 + 4 * u : R;   // past np: reread R, drop it
          const int64_t j = slot_of(k);
          wv[u] = k0 + 4 * u < np ? ml[j * kMlRecord + 1] * merge_weight(ml[j * kMlRecord], big)
                                  : 0.0f;
          const float* sl = po + j * D;
          const int t0 = start + (k - np_pref) * pt;
          const bool half = (!PFX || k >= np_pref) && a.part_half &&
                            min(len, t0 + pt) - t0 >= kHalfPartialMinTokens;
          // 16 bytes at the lane's bf16 position, or 32 at its fp32 one
          const uint4 w0 = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(sl) +
                                                          (half ? 16 : 32) * c);
          const uint4 w1 = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(sl) +
                                                          (half ? 16 : 32) * c + 16);
          if (half) {
            Elem<uint16_t>::unpack(w0, v[u]);
          } else {
            Elem<float>::unpack(w0, v[u]);
            Elem<float>::unpack(w1, v[u] + 4);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc8[e] = fmaf(wv[u], v[u][e], acc8[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc8[e] += xor_lanes<16>(acc8[e]);
        acc8[e] += xor_lanes<32>(acc8[e]);
      }
      // lane (R, c) keeps dims 8c + 2R, 8c + 2R + 1 of the sum, which the
      // store below expects as dims 2 * lane', 2 * lane' + 1 of lane'
      // = 4c + R
      const float d0 = acc8[2 * R], d1 = acc8[2 * R + 1];
      const int src = ((lane & 3) << 4) | (lane >> 2);    // lane (R', c') with 4c' + R' = lane
      o[0] = __shfl(d0, src);
      o[1] = __shfl(d1, src);
    } else {
      for (int k = 0; k < np; ++k) {
        const int64_t j = slot_of(k);
        const float wj = ml[j * kMlRecord + 1] * merge_weight(ml[j * kMlRecord], big);
        float f[DPL];
        load_part(k, f);
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = fmaf(wj, f[e], o[e]);
      }
    }
  }
  T* out = reinterpret_cast<T*>(a.out) + ((int64_t)i * a.num_q_heads + hq) * D + lane * DPL;
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
#pragma unroll
  for (int k = 0; k < DPL; ++k) Elem<T>::store(out + k, o[k] * inv);
}

// The reduce for bf16 output, head dim 128 and 4 query heads per KV head:
// one wave per (sequence, KV head). Lane l serves head l / 16 of the group
// and dims 8 (l % 16) .. + 7, so the group's statistics record is read once
// and a partial slice is one 16-byte (bf16) or 32-byte (fp32) read per lane.
// Lane c of a row holds the statistics of partition c of each batch of 16.
// PFX: the shared-prefix decode's slots, as in decode_reduce<PFX>: first the
// prefix pass's (fp32), then the walk's own partitions from slot0.
template <bool PFX>
__global__ __launch_bounds__(kReduceWaves * 64) void decode_reduce_g4(DecodeArgs a) {
  constexpr int D = 128, G = 4, R = kReduceFast;
  static_assert(R == 16, "one partition per lane of a 16-lane row");
  const int unit = blockIdx.x * kReduceWaves + (threadIdx.x >> 6);
  if (unit >= a.num_seqs * a.num_kv_heads) return;
  const int g = unit % a.num_kv_heads, i = unit / a.num_kv_heads;
  int len = a.seq_lens[i];
  len = len < 0 ? 0 : min(len, a.len_cap);
  if (PFX && len == 0) return;
  const int pt = a.part_tokens;
  const int start = PFX ? walk_start(a, i, len, false) : 0;
  const int np_pref = PFX ? (start + a.prefix_part_tokens - 1) / a.prefix_part_tokens : 0;
  const int np = np_pref + (len - start + pt - 1) / pt;
  if (!PFX && np <= 1) return;                   // written by the partition kernel
  const int64_t stride = PFX ? a.slot_stride : a.max_parts;
  auto slot_of = [&](int k) { return PFX && k >= np_pref ? a.slot0 + (k - np_pref) : k; };
  const int lane = threadIdx.x & 63, h = lane >> 4, c = lane & 15;
  const float* rec = a.part_ml + ((int64_t)i * a.num_kv_heads + g) * stride * kMlRecord + 2 * h;
  const int64_t row = (int64_t)i * a.num_q_heads + g * G + h;
  const char* po = reinterpret_cast<const char*>(a.part_o) + row * stride * D * 4;
  float o[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  // batch of partitions j0 .. j0 + 15 with weights wj (lane c: partition j0 + c)
  auto accumulate = [&](int j0, float wj) {
    // every load of the batch first; partitions past np (a wave-uniform
    // test) load nothing
    uint4 w0[R], w1[R];
    bool half[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int j = j0 + u;
      const int t0 = start + (j - np_pref) * pt;
      half[u] = (!PFX || j >= np_pref) && a.part_half &&
                min(len, t0 + pt) - t0 >= kHalfPartialMinTokens;
      w0[u] = w1[u] = make_uint4(0u, 0u, 0u, 0u);
      if (j < np) {
        const char* sl = po + (int64_t)slot_of(j) * D * 4 + (half[u] ? 16 : 32) * c;
        w0[u] = *reinterpret_cast<const uint4*>(sl);
        w1[u] = *reinterpret_cast<const uint4*>(sl + 16);
      }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const float w = __shfl(wj, (lane & 48) | u);
      float f[8];
      Elem<uint16_t>::unpack(w0[u], f);
      const float v[8] = {half[u] ? f[0] : __uint_as_float(w0[u].x),
                          half[u] ? f[1] : __uint_as_float(w0[u].y),
                          half[u] ? f[2] : __uint_as_float(w0[u].z),
                          half[u] ? f[3] : __uint_as_float(w0[u].w),
                          half[u] ? f[4] : __uint_as_float(w1[u].x),
                          half[u] ? f[5] : __uint_as_float(w1[u].y),
                          half[u] ? f[6] : __uint_as_float(w1[u].z),
                          half[u] ? f[7] : __uint_as_float(w1[u].w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(w, v[e], o[e]);
    }
  };
  auto row_max = [](float x) {
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
  };
  float wsum;
  if (np <= R) {
    // every read up front
    const float mj = c < np ? rec[(int64_t)slot_of(c) * kMlRecord] : -INFINITY;
    const float lj = c < np ? rec[(int64_t)slot_of(c) * kMlRecord + 1] : 0.0f;
    const float wj = lj * merge_weight(mj, row_max(mj));
    accumulate(0, wj);
    wsum = wj;
  } else {
    float big = -INFINITY;
    for (int j0 = 0; j0 < np; j0 += R)
      if (j0 + c < np) big = fmaxf(big, rec[(int64_t)slot_of(j0 + c) * kMlRecord]);
    big = row_max(big);
    wsum = 0.0f;
    for (int j0 = 0; j0 < np; j0 += R) {
      const int j = j0 + c;
      const float* rj = rec + (int64_t)slot_of(j) * kMlRecord;
      const float wj = j < np ? rj[1] * merge_weight(rj[0], big) : 0.0f;
      accumulate(j0, wj);
      wsum += wj;
    }
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + row * D + 8 * c;
  store4<uint16_t>(out, o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  store4<uint16_t>(out + 4, o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
}

// ---------------------------------------------------------------------------
// Slot write and block copy
// ---------------------------------------------------------------------------
// One thread per 16-byte chunk of a (token, head) row, K and V together.
// Table and length upkeep of an appended token (one thread per token): the
// token of sequence t lands at position p = seq_lens[t], so the block of its
// slot becomes table entry p / bs (a new block, a copy-on-write
// replacement, or the entry already there) and the length becomes p + 1.
// A position outside the table, or a slot whose offset is not p % bs, is
// flagged and leaves table and length alone.
__device__ __forceinline__ void append_upkeep(const AppendArgs& ap, int64_t t, int64_t slot,
                                              int block_size) {
  const int p = ap.seq_lens[t];
  if (p < 0 || p / block_size >= ap.max_blocks || slot % block_size != p % block_size) {
    flag_error(kErrSlot);
    return;
  }
  ap.block_tables[t * ap.max_blocks + p / block_size] = (int32_t)(slot / block_size);
  ap.seq_lens[t] = p + 1;
}

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)a.num_kv_heads * a.row_chunks;
  if (idx >= per_token * a.num_tokens) return;
  const int64_t t = idx / per_token;
  const int64_t rem = idx - t * per_token;
  const int h = (int)(rem / a.row_chunks);
  const int c = (int)(rem - (int64_t)h * a.row_chunks);
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    if (rem == 0) flag_error(kErrSlot);
    return;
  }
  if (a.append.block_tables && rem == 0) append_upkeep(a.append, t, slot, a.block_size);
  const int64_t b = slot / a.block_size, o = slot - b * a.block_size;
  const int64_t dst = ((b * a.num_kv_heads + h) * a.block_size + o) * a.row_chunks + c;
  const int64_t src = idx;  // [T][Hkv][row_chunks] is exactly the thread order
  reinterpret_cast<uint4*>(a.k_pool)[dst] = reinterpret_cast<const uint4*>(a.k)[src];
  reinterpret_cast<uint4*>(a.v_pool)[dst] = reinterpret_cast<const uint4*>(a.v)[src];
}

// FP8 E4M3 code of the exact quotient x / s (s > 0 and finite): the nearest
// code, ties to the even mantissa, saturating at +-448, NaN to 0x7F with x's
// sign. The quotient is formed in double, which decides every case as the
// exact quotient would: a midpoint between two codes has at most 5
// significant bits, so the quotient of two floats is either such a midpoint
// exactly or at least 2^-29 of its size away from it, far more than one
// double rounding moves it. In the normal range the double's mantissa is
// then rounded to 3 bits on its bit pattern (carry into the exponent
// included) and the exponent rebased from 1023 to 7; below 2^-6 the code is
// the subnormal count round(x / s * 2^9), ties to even.
__device__ __forceinline__ uint32_t e4m3_code_of_quotient(float x, float s) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  if (x != x) return 0x7fu | sign;
  const double a = fabs((double)x) / (double)s;
  if (a >= 448.0) return 0x7eu | sign;
  if (a < 0.015625) return (uint32_t)__builtin_rint(a * 512.0) | sign;
  const uint64_t b = (uint64_t)__double_as_longlong(a);
  const uint64_t r = b + 0xffffffffffffull + ((b >> 49) & 1u);
  return (uint32_t)((r >> 49) - (1016ull << 3)) | sign;
}

// One thread per 8 elements of a (token, head) row, K and V together: 16
// bytes of bf16 in, 8 bytes of codes out.
__global__ __launch_bounds__(256) void reshape_and_cache_e4m3_kernel(CacheArgs8 a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = (int64_t)a.num_kv_heads * a.row_groups;
  if (idx >= per_token * a.num_tokens) return;
  const int64_t t = idx / per_token;
  const int64_t rem = idx - t * per_token;
  const int h = (int)(rem / a.row_groups);
  const int c = (int)(rem - (int64_t)h * a.row_groups);
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    if (rem == 0) flag_error(kErrSlot);
    return;
  }
  if (a.append.block_tables && rem == 0) append_upkeep(a.append, t, slot, a.block_size);
  const int64_t b = slot / a.block_size, o = slot - b * a.block_size;
  const int64_t dst = ((b * a.num_kv_heads + h) * a.block_size + o) * a.row_groups + c;
  for (int pool = 0; pool < 2; ++pool) {
    const uint4 x = reinterpret_cast<const uint4*>(pool ? a.v : a.k)[idx];
    const float sc = pool ? a.v_scale : a.k_scale;
    float f[8];
    Elem<uint16_t>::unpack(x, f);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e >> 2] |= e4m3_code_of_quotient(f[e], sc) << (8 * (e & 3));
    reinterpret_cast<uint2*>(pool ? a.v_pool : a.k_pool)[dst] = make_uint2(w[0], w[1]);
  }
}

// grid.x = pair, grid.z = pool (0 K, 1 V); grid.y strides over the block.
// Four 16-byte loads per thread are in flight before their stores, which
// matters when one side is host memory reached over the host link.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int n = blockIdx.x;
  const int64_t src = a.pairs[2 * n], dst = a.pairs[2 * n + 1];
  if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) {
    if (blockIdx.y == 0 && threadIdx.x == 0 && blockIdx.z == 0) flag_error(kErrCopyPair);
    return;
  }
  const uint4* s = reinterpret_cast<const uint4*>(blockIdx.z == 0 ? a.src_k : a.src_v) +
                   src * a.block_chunks;
  uint4* d = reinterpret_cast<uint4*>(blockIdx.z == 0 ? a.dst_k : a.dst_v) + dst * a.block_chunks;
  const int64_t step = (int64_t)gridDim.y * blockDim.x;
  int64_t k = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  for (; k + 3 * step < a.block_chunks; k += 4 * step) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = s[k + u * step];
#pragma unroll
    for (int u = 0; u < 4; ++u) d[k + u * step] = v[u];
  }
  for (; k < a.block_chunks; k += step) d[k] = s[k];
}


// ---------------------------------------------------------------------------
// Multi-token queries (prefill chunk / speculative tokens) on matrix cores
// ---------------------------------------------------------------------------
// Unit of work: one wave per (sequence, KV head, tile of 16 query rows); a
// query row is a (query token, head of the group) pair, row = token * G + h,
// so a tile holds 16 / G consecutive tokens. Positions are walked 16 at a
// time (a "chunk"), up to the tile's last token, through the block table.
// Lane l: R = l / 16, c = l % 16.
//   S^T = K Q^T (v_mfma_f32_16x16x32_bf16): A = K rows of the chunk (lane:
//     token c, dims 8R + 32s ..), B = the tile's query rows (lane: row c,
//     same dims); lane gets S[row c][tokens 4R .. 4R+3].
//   causal mask per row, online softmax per row (row c's 16 scores sit in
//     lanes c, c+16, c+32, c+48: reduced with 16/32-lane swaps).
//   O += P V (v_mfma_f32_16x16x32_bf16, 8 tiles of 16 dims) once per pair of
//     chunks: A = P exactly as the softmax leaves it (lane: row c, positions
//     4R .. 4R+3 of both chunks = its 8 k-slots; split into two bf16 terms,
//     so two products per tile), B = V^T[dim 16t + c][the same 8 positions],
//     one 16-byte read of the pair's V staged transposed in LDS (each lane
//     writes its 4 positions x 8 dims as 8-byte column pieces); lane gets
//     O[rows 4R .. 4R+3][dim 16t + c].
// Each wave owns its LDS buffers and its unit, so waves never wait for one
// another; K/V of chunk c+1 are issued before chunk c is computed.



// p as two bf16 terms hi + lo (lo = the bf16 rounding of p - hi), 8 values
// per operand: ~16 significant bits instead of bf16's 8.
__device__ __forceinline__ void split_bf16x8(const float (&p)[8], uint4& hi, uint4& lo) {
  uint32_t hb[4], lb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hb[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
    lb[e] = pack_bf16x2(p[2 * e] - __uint_as_float(hb[e] << 16),
                        p[2 * e + 1] - __uint_as_float(hb[e] & 0xffff0000u));
  }
  hi = make_uint4(hb[0], hb[1], hb[2], hb[3]);
  lo = make_uint4(lb[0], lb[1], lb[2], lb[3]);
}

constexpr int kMqWaves = 4;
// Staged V^T: row = dim, 40 bf16 per row (32 positions + 8 pad). The four
// 16-byte chunks of rows 64..127 sit in the order 2, 3, 0, 1 (chunk index
// XOR 2): the transposing 8-byte writes of a wave cover rows 8c + k for
// c = 0..15, which without the swap fall on only 16 of the 64 LDS banks.
constexpr int kMqVtRow = 40;
__device__ __forceinline__ int mq_vt_chunk(int row, int chunk) { return chunk ^ ((row >> 5) & 2); }

__device__ __forceinline__ uint16_t bf16_bits(float f) { return to_bf16(f); }

// The per-tile kernel's work for workgroup (bx, by = KV head, bz = sequence
// or group), staging V^T in s_vt.
template <int BS, int G, int NWV = kMqWaves>
__device__ __forceinline__ void mq_tiles(const MqArgs& a, int bx, int by, int bz,
                                         uint16_t (*s_vt)[128][kMqVtRow]) {
  constexpr int D = 128, ROW = 256;
  constexpr int64_t kHeadBytes = (int64_t)BS * ROW;
  static_assert(BS % 16 == 0 && 16 % G == 0, "whole chunks per block, whole tokens per tile");

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = lane >> 4, c = lane & 15;
  const int g = by;
  // units (tile, context partition), partition fastest, one per wave; in
  // decode mode over a host work plan, unit u = plan entry u (sequence,
  // partition, length), one tile each, and the grid holds only those
  const int unit = bx * NWV + w;
  int i = bz, part, tile, plan_len = -1;
  if (a.plan) {
    if (unit >= a.num_units) return;
    const int4 e = reinterpret_cast<const int4*>(a.plan)[unit];
    i = e.x;
    part = e.y;
    tile = 0;
    plan_len = e.z;
    const int np = a.part_tokens > 0 ? (plan_len + a.part_tokens - 1) / a.part_tokens : 1;
    if ((unsigned)i >= (unsigned)a.num_seqs || (unsigned)plan_len > (unsigned)a.len_cap ||
        part < 0 || part >= (np > 1 ? np : 1)) {
      if (lane == 0) flag_error(kErrPlan);
      return;
    }
  } else {
    part = unit % a.max_parts;
    tile = unit / a.max_parts;
  }

  // validate the sequence's length and query range (device-resident). The
  // walk covers positions [wstart, npos) of the sequence (the tile's last
  // row sees npos - 1); row c sees positions up to pos_c (below).
  int L, q0, tq, wstart = 0;
  int64_t trow_base = (int64_t)i * a.max_blocks;
  const int mode = a.mode ? a.mode : (a.decode_mode ? 1 : 0);
  if (mode == 1 || mode == 3) {
    // pa_decode: token i; a length outside [0, len_cap] is clamped and
    // flagged, and an empty sequence gets zero rows (a plan's lengths were
    // checked above)
    L = plan_len >= 0 ? plan_len : a.seq_lens[i];
    q0 = i;
    tq = 1;
    if (L < 0 || L > a.len_cap) {
      if (lane == 0 && g == 0 && unit == 0) flag_error(kErrSeqLen);
      L = L < 0 ? 0 : a.len_cap;
    }
    if (L == 0) {
      if (a.plan ? part == 0 : unit == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * R + r < G) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) +
                            ((int64_t)i * a.num_q_heads + g * G + 4 * R + r) * D + c;
#pragma unroll
            for (int t2 = 0; t2 < 8; ++t2) dst[16 * t2] = 0;
          }
      return;
    }
    if (mode == 3) {
      // the positions after the shared prefix
      wstart = a.prefix_lens[i];
      if (wstart < 0 || wstart > L || wstart > a.max_prefix || wstart % BS != 0) {
        if (lane == 0 && g == 0 && unit == 0) flag_error(kErrPrefix);
        wstart = 0;
      }
      if (wstart == L) return;
    }
  } else if (mode == 2) {
    // one group: its sequences are the query tokens, the first one's table
    // and prefix length serve all of them, every row sees the whole prefix
    q0 = a.group_start[i];
    tq = a.group_start[i + 1] - q0;
    if (q0 < 0 || tq < 0 || q0 + tq > a.num_tokens || tq > a.max_query_len) {
      if (lane == 0 && g == 0 && unit == 0) flag_error(kErrPrefix);
      return;
    }
    if (tq == 0) return;
    L = a.prefix_lens[q0];
    if (L < 0 || L > a.len_cap || L > a.max_prefix || L % BS != 0) {
      if (lane == 0 && g == 0 && unit == 0) flag_error(kErrPrefix);
      return;
    }
    if (L == 0) return;
    trow_base = (int64_t)q0 * a.max_blocks;
    if (g == 0 && unit == 0) {
      // every member must share the prefix: same length, same blocks, and
      // at least that many cached positions
      bool bad = false;
      const int nb = L / BS;
      for (int k = lane; k < (tq - 1) * nb; k += 64) {
        const int sm = q0 + 1 + k / nb, blk = k % nb;
        bad |= a.block_tables[(int64_t)sm * a.max_blocks + blk] != a.block_tables[trow_base + blk];
      }
      for (int sm = q0 + lane; sm < q0 + tq; sm += 64)
        bad |= a.prefix_lens[sm] != L || a.seq_lens[sm] < L;
      if (__ballot(bad) != 0 && lane == 0) flag_error(kErrPrefix);
    }
  } else {
    L = a.seq_lens[i];
    q0 = a.query_start[i];
    const int q1 = a.query_start[i + 1];
    tq = q1 - q0;
    if (L < 0 || L > a.len_cap || q0 < 0 || q1 > a.num_tokens || tq < 0 || tq > L ||
        tq > a.max_query_len) {
      if (lane == 0 && g == 0 && bx == 0) flag_error(kErrQuery);
      return;
    }
  }
  const int rows = tq * G;
  if (tile * 16 >= rows) return;
  const int row0 = tile * 16;
  const int t_last = min(tq - 1, (row0 + 15) / G);
  const bool causal = mode <= 1;
  const int npos = causal ? L - tq + t_last + 1 : L;
  // this wave's context partition: positions [pos0, pos1)
  const int nparts =
      a.part_tokens > 0 ? (npos - wstart + a.part_tokens - 1) / a.part_tokens : 1;
  if (part >= nparts) return;
  const int pos0 = wstart + (a.part_tokens > 0 ? part * a.part_tokens : 0);
  const int pos1 = a.part_tokens > 0 ? min(npos, pos0 + a.part_tokens) : npos;
  const int ch0 = pos0 / 16;
  const int nch = (pos1 + 15) / 16 - ch0;
  // the shared-prefix passes always leave partials (merged with the other
  // pass); the per-sequence pass after the prefix pass's slots
  const bool direct = causal && nparts == 1;
  const int slot = (mode == 3 ? a.suffix_slot0 : 0) + part;

  // this lane's query row (column of S^T): token tc, head hc
  const int rc = row0 + c;
  const bool row_ok = rc < rows;
  const int tc = rc / G, hc = rc % G;
  const int pos_c = causal ? L - tq + tc : L - 1;   // last position row c attends to
  bf16x8_t qop[4];
  {
    const int trow = row_ok ? tc : 0;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((int64_t)(q0 + trow) * a.num_q_heads + g * G + hc) * D + 8 * R) * 2;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      uint4 v = row_ok ? ld16(qp, s2 * 64) : make_uint4(0, 0, 0, 0);
      qop[s2] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  const int64_t blk_bytes = kHeadBytes * a.num_kv_heads;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + g * kHeadBytes;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + g * kHeadBytes;
  const uint32_t k_off = (uint32_t)(c * ROW + R * 16);
  const uint32_t v_off = (uint32_t)(4 * R * ROW + c * 16);

  float m = -INFINITY, lsum = 0.0f;             // softmax state of row c
  f32x4_t acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int win = 0; win < nch; win += 64) {
    const int cnt = min(64, nch - win);
    int ids = 0;
    if (lane < cnt)
      ids = checked_id(a.block_tables, a.num_blocks, trow_base, ((ch0 + win + lane) * 16) / BS);
    auto issue = [&](KVChunk& buf, int t) {
      const int phys = __builtin_amdgcn_readlane(ids, t);
      // K with the plain policy (its lines are read in halves, see
      // load_kv_chunk): decode at group 8 487-492 -> 477 us, speculative
      // tokens over split contexts 499 -> 485 us; V streams
      load_kv_chunk<BS, kKvStream, kKvCached>(buf, kbase, vbase, blk_bytes, phys,
                                              ((ch0 + win + t) * 16) % BS, k_off, v_off, true);
    };
    KVChunk b0, b1;
    // chunks go in pairs (32 positions: one P.V step); the first chunk's
    // scores wait in sc_a while the second is loaded
    f32x4_t sc_a = {0.0f, 0.0f, 0.0f, 0.0f};
    auto pair_step = [&](const f32x4_t& s0, const f32x4_t& s1, int tok0, bool has_b) {
      // lane's 8 scores of row c: positions tok0 + 16h + 4R + r = k-slot 4h + r
      float sv[8];
      float bm = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = (h ? s1[r] : s0[r]) * a.qscale;
          const bool ok = row_ok && (h == 0 || has_b) && (tok0 + 16 * h + 4 * R + r <= pos_c);
          sv[4 * h + r] = ok ? v : -INFINITY;
          bm = fmaxf(bm, sv[4 * h + r]);
        }
      bm = fmaxf(bm, xor_lanes<16>(bm));
      bm = fmaxf(bm, xor_lanes<32>(bm));
      const float mn = bm > m + kLazyMax ? bm : m;
      const float alpha = mn == m ? 1.0f : exp2_fast(m - mn);
      m = mn;
      float p[8], ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = sv[e] == -INFINITY ? 0.0f : exp2_fast(sv[e] - mn);
        ps += p[e];
      }
      ps += xor_lanes<16>(ps);
      ps += xor_lanes<32>(ps);
      lsum = lsum * alpha + ps;
      // rescale output rows 4R + r by their rows' alpha (held by lane 4R + r)
      if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, 4 * R + r);
#pragma unroll
          for (int t2 = 0; t2 < 8; ++t2) acc[t2][r] *= ar;
        }
      }
      uint4 phi, plo;
      split_bf16x8(p, phi, plo);
      __builtin_amdgcn_wave_barrier();   // the staged V^T rows are complete (in-order per wave)
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) {
        const int row = 16 * t2 + c;
        const bf16x8_t vb = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&s_vt[w][row][8 * mq_vt_chunk(row, R)]));
        acc[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, phi), vb,
                                                          acc[t2], 0, 0, 0);
        acc[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, plo), vb,
                                                          acc[t2], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
    };
    // stage V of half h of the pair transposed: V^T row = dim, slot 8R + 4h + r
    // holds position 16h + 4R + r; rows past the tile's last position are
    // zeros, so that slack slots (which may hold anything, NaN included)
    // never meet the zero weights
    auto stage_vt = [&](const KVChunk& cur, int h, bool zero) {
      uint32_t v[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint4 x = zero ? make_uint4(0, 0, 0, 0) : cur.v[r];
        v[r][0] = x.x;
        v[r][1] = x.y;
        v[r][2] = x.z;
        v[r][3] = x.w;
      }
      // rows 8c .. 8c + 7 share one chunk order
      const int slot = 8 * mq_vt_chunk(8 * c, R) + 4 * h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 lo = make_uint2(pack_low_halves(v[0][e], v[1][e]),
                                    pack_low_halves(v[2][e], v[3][e]));
        const uint2 hi = make_uint2(pack_high_halves(v[0][e], v[1][e]),
                                    pack_high_halves(v[2][e], v[3][e]));
        *reinterpret_cast<uint2*>(&s_vt[w][8 * c + 2 * e][slot]) = lo;
        *reinterpret_cast<uint2*>(&s_vt[w][8 * c + 2 * e + 1][slot]) = hi;
      }
    };
    auto step = [&](KVChunk& cur, int t) {
      const int chunk = ch0 + win + t;
      const int tok0 = chunk * 16;
      const int h = (win + t) & 1;
      if (tok0 + 16 > npos) {
        // zero the rows of this chunk past npos
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (tok0 + 4 * R + jj >= npos) cur.v[jj] = make_uint4(0, 0, 0, 0);
      }
      stage_vt(cur, h, false);
      f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[s2]),
                                                     qop[s2], sc, 0, 0, 0);
      if (h == 0) {
        sc_a = sc;
        if (t + 1 >= cnt) {
          // a chunk without a partner: its second half is empty
          stage_vt(cur, 1, true);
          pair_step(sc_a, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, tok0, false);
        }
      } else {
        pair_step(sc_a, sc, tok0 - 16, true);
      }
    };
    issue(b0, 0);
    for (int t = 0;;) {
      issue(b1, t + 1 < cnt ? t + 1 : t);
      step(b0, t);
      if (++t >= cnt) break;
      issue(b0, t + 1 < cnt ? t + 1 : t);
      step(b1, t);
      if (++t >= cnt) break;
    }
  }
  // out[row] = O[row] / l[row]; lane holds rows 4R + r, dims 16 t + c. With
  // several partitions: the normalised partial output (bf16) and the row's
  // (max, exp-sum), merged by multi_query_reduce.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lr = __shfl(lsum, 4 * R + r);
    const float mr = __shfl(m, 4 * R + r);
    const int row = row0 + 4 * R + r;
    if (row >= rows) continue;
    const int t = row / G, h = row % G;
    const int64_t qrow = (int64_t)(q0 + t) * a.num_q_heads + g * G + h;
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
    const int64_t pslot = qrow * (a.slot_stride ? a.slot_stride : a.max_parts) + slot;
    if (direct || a.part_half) {
      uint16_t* dst = direct ? reinterpret_cast<uint16_t*>(a.out) + qrow * D + c
                             : reinterpret_cast<uint16_t*>(a.part_o) + pslot * D + c;
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) dst[16 * t2] = bf16_bits(acc[t2][r] * inv);
    } else {
      float* dst = reinterpret_cast<float*>(a.part_o) + pslot * D + c;
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) dst[16 * t2] = acc[t2][r] * inv;
    }
    if (!direct && c == 0) {
      // per row, or pa_decode's records: (sequence, KV head, slot), the
      // group's heads side by side
      float* ml = a.ml_records
                      ? a.part_ml + (((int64_t)(q0 + t) * a.num_kv_heads + g) *
                                         (a.slot_stride ? a.slot_stride : a.max_parts) + slot) *
                                        kMlRecord + 2 * h
                      : a.part_ml + pslot * 2;
      ml[0] = mr;
      ml[1] = lr;
    }
  }
}

template <int BS, int G>
__global__ __launch_bounds__(kMqWaves * 64, 3) void multi_query_mfma(MqArgs a) {
  __shared__ __align__(16) uint16_t s_vt[kMqWaves][128][kMqVtRow];
  mq_tiles<BS, G>(a, blockIdx.x, blockIdx.y, blockIdx.z, s_vt);
}

// Shared-prefix decode, both passes in one launch so that they run side by
// side: workgroups 0 .. n_prefix - 1 are the prefix pass (the per-tile kernel
// over (tile/partition group, KV head, group)), the rest the per-sequence
// walks (pa_decode's matrix-core kernel after the prefix).
struct CascadeArgs {
  MqArgs pre;
  DecodeArgs walk;
  int32_t n_prefix;      // workgroups of the prefix pass
  int32_t pre_gx;        // its grid: pre_gx x num_kv_heads x num_groups
};

// Waves per workgroup of the shared-prefix decode: one 16-row tile each in
// the prefix pass, two per (sequence, KV head, partition) unit in the walks
// (as the decode kernel on large grids: twice the workgroups of a 4-wave
// walk, which evens out the end of the grid; a 32,768-position sequence
// makes 64 units per KV head).
constexpr int kCascadeWaves = 2;

template <int BS, int G>
__global__ __launch_bounds__(kCascadeWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
void shared_prefix_decode(CascadeArgs ca) {
  __shared__ __align__(16) uint16_t s_vt[kCascadeWaves][128][kMqVtRow];
  const int id = blockIdx.x;
  if (id < ca.n_prefix) {
    const int bx = id % ca.pre_gx, r = id / ca.pre_gx;
    mq_tiles<BS, G, kCascadeWaves>(ca.pre, bx, r % ca.pre.num_kv_heads,
                                   r / ca.pre.num_kv_heads, s_vt);
    return;
  }
  PartitionWork wk;
  if (!setup_partition<uint16_t, 128, BS, G, kCascadeWaves, true>(ca.walk, wk, id - ca.n_prefix))
    return;
  mfma_unit<BS, G, kCascadeWaves, false, true>(ca.walk, wk);
}

// Merge of the context partitions of pa_multi_query's split form: one wave
// per (sequence, query token, query head) row, kMqWaves rows per workgroup;
// the partition count of a row is that of its 16-row tile, as in
// multi_query_mfma.
template <int G>
__global__ __launch_bounds__(kMqWaves * 64) void multi_query_reduce(MqArgs a) {
  constexpr int D = 128, DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.y;
  const int lr = blockIdx.x * kMqWaves + (threadIdx.x >> 6);   // row within the sequence
  int L = a.seq_lens[i];
  int q0, tq;
  int np_pref = 0, start = 0;    // shared-prefix decode: the prefix pass's slots
  if (a.decode_mode || a.mode == 3) {
    q0 = i;
    tq = 1;
    L = L < 0 ? 0 : min(L, a.len_cap);           // as multi_query_mfma
    if (L == 0) return;
    if (a.mode == 3) {
      start = a.prefix_lens[i];
      if (start < 0 || start > L || start > a.max_prefix || start % a.block_size != 0) start = 0;
      np_pref = (start + a.prefix_part_tokens - 1) / a.prefix_part_tokens;
    }
  } else {
    q0 = a.query_start[i];
    const int q1 = a.query_start[i + 1];
    tq = q1 - q0;
    if (L < 0 || L > a.len_cap || q0 < 0 || q1 > a.num_tokens || tq < 0 || tq > L ||
        tq > a.max_query_len)
      return;                                    // flagged by multi_query_mfma
  }
  if (lr >= tq * a.num_q_heads) return;
  const int t = lr / a.num_q_heads, hq = lr % a.num_q_heads;
  const int row0 = ((t * G + hq % G) / 16) * 16;  // first row of its tile
  const int t_last = min(tq - 1, (row0 + 15) / G);
  const int npos = L - tq + t_last + 1;
  // partial k of the row sits in slot k, or for shared-prefix decode the
  // prefix pass's np_pref slots come first, then the per-sequence pass's
  const int np = a.mode == 3 ? np_pref + (L - start + a.part_tokens - 1) / a.part_tokens
                             : (npos + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1 && a.mode != 3) return;
  auto slot = [&](int k) { return a.mode == 3 && k >= np_pref ? a.suffix_slot0 + k - np_pref : k; };
  const int64_t qrow = (int64_t)(q0 + t) * a.num_q_heads + hq;
  const int64_t stride = a.slot_stride ? a.slot_stride : a.max_parts;
  const float* ml = a.part_ml + qrow * stride * 2;
  const int64_t po = qrow * stride * D;
  float mj = -INFINITY, lj = 0.0f;
  for (int k = lane; k < np; k += 64) {
    const int j = slot(k);
    const float m2 = ml[2 * j], l2 = ml[2 * j + 1];
    const float big = fmaxf(mj, m2);
    lj = lj * merge_weight(mj, big) + l2 * merge_weight(m2, big);
    mj = big;
  }
  float big = mj;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) big = fmaxf(big, __shfl_xor(big, off));
  float wsum = lj * merge_weight(mj, big);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
  float o[DPL] = {0.0f, 0.0f};
  for (int k = 0; k < np; ++k) {
    const int j = slot(k);
    const float wj = ml[2 * j + 1] * merge_weight(ml[2 * j], big);
    float f[DPL];
    if (a.part_half)
      load_elems<uint16_t, DPL>(reinterpret_cast<const uint16_t*>(a.part_o) + po + (int64_t)j * D +
                                    lane * DPL, f);
    else
      load_elems<float, DPL>(reinterpret_cast<const float*>(a.part_o) + po + (int64_t)j * D +
                                 lane * DPL, f);
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = fmaf(wj, f[k], o[k]);
  }
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + qrow * D + lane * DPL;
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
#pragma unroll
  for (int k = 0; k < DPL; ++k) out[k] = bf16_bits(o[k] * inv);
}


// ---------------------------------------------------------------------------
// Multi-token queries, many rows per (sequence, KV head): one workgroup of 8
// waves (one per CU: 2 per SIMD) per tile of 256 query rows, 32 rows per wave,
// on 32x32x16 matrix products. Positions are walked 64 at a time (a "block");
// each block's K rows and V rows are read from the pool once per workgroup and
// staged in LDS, each of the 512 threads loading and staging 2 positions of
// one 16-byte column of K and of V:
//   K as rows (272-byte stride: the 16 lanes of a read group hit distinct
//     banks); the A operand of S^T = K Q^T is a 16-byte LDS read;
//   V transposed (V^T, dims as rows, 144-byte stride), with the positions of
//     each 16-position group permuted so that the 8 positions a lane
//     contributes to one P.V step are contiguous: the A operand of
//     O^T += V^T P^T is a 16-byte LDS read too.
// Lane l: n = l % 32 (the wave's query row n), hh = l / 32. Each S^T tile
// (32 positions x 32 rows) leaves lane (hh, n) 16 scores of row n, at
// positions 8 (v / 4) + 4 hh + v % 4 (v = 0 .. 15); the 8 of them in one
// 16-position group are exactly the lane's k-slots (8 hh ..) of the B operand
// (P^T) of a P.V step, so P goes from the softmax to the matrix cores without
// leaving the lane: in fp16, with V^T staged in fp16 (11 significant bits, 8x
// finer than bf16; for tiles whose V values stay within +-kFaF16VMax), or, on
// the exact pass, as two bf16 terms p = hi + lo (~16 significant bits) against
// bf16 V^T. With rows in lanes the softmax is lane-local but for one 32-lane
// swap per block (the row maximum) and one at the end (the row sum). The next
// block's K/V loads are issued before the current block is computed.
// Workgroup ids: every tile of one (sequence, KV head) lands on the same XCD
// (XCD = id % 8), so the tiles share that XCD's L2 copy of the context;
// heavier (later) tiles first.
#ifndef PA_FA_WAVES
#define PA_FA_WAVES 8
#endif
constexpr int kFaWaves = PA_FA_WAVES;   // waves per workgroup, 32 query rows each
constexpr int kFaRows = 32 * kFaWaves;  // query rows per workgroup
constexpr int kFaMinRows = 128;         // rows per KV head from which calls take this kernel
constexpr int kFaPos = 64;       // positions per block
// positions of one staged block per loader thread (16-byte pieces of K and V)
constexpr int kFaNp = kFaPos * 16 / (kFaWaves * 64);
static_assert(kFaNp == 2 || kFaNp == 4, "4 or 8 waves per workgroup");
constexpr int kFaKRow = 136;     // bf16 elements per staged K row (128 + 8 pad)
constexpr int kFaVRow = 72;      // bf16 elements per staged V^T row (64 + 8 pad)
constexpr int kFaBufs = 2;       // LDS stages of K and V^T (one barrier per block)
// The fp16 pass serves tiles whose context holds V values within
// +-kFaF16VMax only (its weights' rounding then moves an output by at most
// 2^-10 * 2 * kFaF16VMax, and in practice as little as the two-term P does);
// a tile that meets a larger value leaves it to the exact pass.
constexpr float kFaF16VMax = 8.0f;


// Slot of position j (0..63) of a block in a staged V^T row: inside each
// 16-position group, position 8q + 4h + r goes to slot 8h + 4q + r (the
// k-slot order of the 32x32x16 operands).
__device__ __forceinline__ int fa_vt_slot(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

typedef uint16_t FaKStage[kFaPos][kFaKRow];
typedef uint16_t FaVtStage[128][kFaVRow];

// One workgroup's tile. F16: P and V^T in fp16 on v_mfma_f32_32x32x16_f16;
// returns false (and writes nothing) as soon as a staged block holds a V value
// beyond +-kFaF16VMax (infinite ones included). Otherwise P as two bf16 terms
// on the bf16 matrix product, for any input.
template <int BS, int G, bool F16>
__device__ __forceinline__ bool multi_query_fa_tile(const MqArgs& a, FaKStage* s_kb, FaVtStage* s_vtb,
                                                    int* s_big) {
  constexpr int D = 128, ROW = 256;
  constexpr int64_t kHeadBytes = (int64_t)BS * ROW;
  static_assert(BS % 16 == 0 && kFaRows % (2 * 16) == 0 && 16 % G == 0,
                "whole 4-position groups per block, whole tokens per 32-row wave");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup id -> (tile, KV head, sequence)
  const int ntiles = (a.max_query_len * G + kFaRows - 1) / kFaRows;
  const int id = blockIdx.x, x = id & 7, rr = id >> 3;
  const int tile = ntiles - 1 - rr % ntiles;
  const int pair = (rr / ntiles) * 8 + x;
  if (pair >= a.num_seqs * a.num_kv_heads) return true;
  const int g = pair % a.num_kv_heads, i = pair / a.num_kv_heads;

  // validate the sequence's length and query range (device-resident)
  const int L = a.seq_lens[i];
  const int q0 = a.query_start[i], q1 = a.query_start[i + 1];
  const int tq = q1 - q0;
  if (L < 0 || L > a.len_cap || q0 < 0 || q1 > a.num_tokens || tq < 0 || tq > L ||
      tq > a.max_query_len) {
    if (tid == 0 && g == 0 && tile == ntiles - 1) flag_error(kErrQuery);
    return true;
  }
  const int rows = tq * G;
  const int row0 = tile * kFaRows;
  if (row0 >= rows) return true;
  const int t_last = min(tq - 1, (row0 + kFaRows - 1) / G);
  const int npos = L - tq + t_last + 1;          // positions the tile's last token sees
  const int nblk = (npos + kFaPos - 1) / kFaPos;

  // this lane's query row (column n of S^T); lanes n and n + 32 share it
  const int n = lane & 31, hh = lane >> 5;
  const int roww = row0 + 32 * w;
  bf16x8_t qop[8];
  int pos_c;
  {
    const int rc = roww + n;
    const bool ok = rc < rows;
    const int tc = ok ? rc / G : 0, hc = rc % G;
    pos_c = ok ? L - tq + tc : -1;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((int64_t)(q0 + tc) * a.num_q_heads + g * G + hc) * D + 8 * hh) * 2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qop[ks] = __builtin_bit_cast(bf16x8_t, ok ? ld16(qp, ks * 32) : make_uint4(0, 0, 0, 0));
  }
  // every row of this wave sees positions below vis_w (its first row's token)
  const int vis_w = L - tq + min(roww, rows - 1) / G + 1;
  // a negative softmax scale is folded into the sign of q, so the scale
  // applied to the scores is never negative
  const float qs = fabsf(a.qscale);
  if (a.qscale < 0.0f) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 u = __builtin_bit_cast(uint4, qop[ks]);
      u.x ^= 0x80008000u;
      u.y ^= 0x80008000u;
      u.z ^= 0x80008000u;
      u.w ^= 0x80008000u;
      qop[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  // loaders: K thread = (token group tk, 16-byte dim chunk dk), V thread =
  // (token group tv, dim chunk dv); each moves 4 consecutive positions
  constexpr int kTg = kFaPos / kFaNp;    // V loaders per dim chunk
  const int dk = tid & 15, tk = tid >> 4;
  const int tv = tid % kTg, dv = tid / kTg;
  const int64_t blk_bytes = kHeadBytes * a.num_kv_heads;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + g * kHeadBytes;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + g * kHeadBytes;
  const int64_t trow = (int64_t)i * a.max_blocks;
  uint4 kreg[kFaNp], vreg[kFaNp];
  // physical blocks of this thread's K and V positions in block `blk`, read
  // one block ahead of the K/V loads that use them and range-checked only
  // there (a check at the read would make the wave wait for every load
  // issued before it)
  auto block_ids = [&](int blk, int& idk, int& idv) {
    const int pk = blk * kFaPos + kFaNp * tk, pv = blk * kFaPos + kFaNp * tv;
    idk = pk < npos ? a.block_tables[trow + pk / BS] : 0;
    idv = pv < npos ? a.block_tables[trow + pv / BS] : 0;
  };
  auto fetch = [&](int blk, int idk, int idv) {
    const int pk = blk * kFaPos + kFaNp * tk, pv = blk * kFaPos + kFaNp * tv;
    if ((unsigned)idk >= (unsigned)a.num_blocks || (unsigned)idv >= (unsigned)a.num_blocks) {
      flag_error(kErrBlockId);
      idk = (unsigned)idk >= (unsigned)a.num_blocks ? 0 : idk;
      idv = (unsigned)idv >= (unsigned)a.num_blocks ? 0 : idv;
    }
    const char* kp = kbase + (int64_t)idk * blk_bytes + (pk % BS) * ROW + 16 * dk;
    const char* vp = vbase + (int64_t)idv * blk_bytes + (pv % BS) * ROW + 16 * dv;
    if ((blk + 1) * kFaPos <= npos) {      // every position of the block is cached
#pragma unroll
      for (int r = 0; r < kFaNp; ++r) {
        kreg[r] = ld16(kp, r * ROW);
        vreg[r] = ld16(vp, r * ROW);
      }
    } else {
#pragma unroll
      for (int r = 0; r < kFaNp; ++r) {
        kreg[r] = pk + r < npos ? ld16(kp, r * ROW) : make_uint4(0, 0, 0, 0);
        vreg[r] = pv + r < npos ? ld16(vp, r * ROW) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // V^T is staged as loaded (bf16, two-term path) or converted to fp16
  // (round to nearest: exact for every bf16 value below 2^16 in magnitude)
  // stage(buf, b): block b into LDS buffer buf; on the fp16 pass a thread
  // that staged a V value beyond +-kFaF16VMax stamps the buffer with b
  auto stage = [&](int buf, int b) {
    uint16_t(*s_k)[kFaKRow] = s_kb[buf];
    uint16_t(*s_vt)[kFaVRow] = s_vtb[buf];
    float vmax = 0.0f;
#pragma unroll
    for (int r = 0; r < kFaNp; ++r)
      *reinterpret_cast<uint4*>(&s_k[kFaNp * tk + r][8 * dk]) = kreg[r];
    const int slot = fa_vt_slot(kFaNp * tv);
    if constexpr (kFaNp == 2) {
      // dims 8 dv + 2e (low halves) and + 2e + 1 (high halves) of 2 positions
      const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vreg[kFaNp - 1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lo, hi;
        if constexpr (F16) {
          const float a0 = __uint_as_float(v0[e] << 16), a1 = __uint_as_float(v1[e] << 16);
          const float b0 = __uint_as_float(v0[e] & 0xffff0000u), b1 = __uint_as_float(v1[e] & 0xffff0000u);
          lo = pack_f16x2(a0, a1);
          hi = pack_f16x2(b0, b1);
          vmax = max3_abs(vmax, a0, a1);
          vmax = max3_abs(vmax, b0, b1);
        } else {
          lo = pack_low_halves(v0[e], v1[e]);
          hi = pack_high_halves(v0[e], v1[e]);
        }
        *reinterpret_cast<uint32_t*>(&s_vt[8 * dv + 2 * e][slot]) = lo;
        *reinterpret_cast<uint32_t*>(&s_vt[8 * dv + 2 * e + 1][slot]) = hi;
      }
      if constexpr (F16) {
        if (vmax > kFaF16VMax) s_big[buf] = b;
      }
    } else {
    const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
    const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vreg[1 % kFaNp]);
    const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&vreg[2 % kFaNp]);
    const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&vreg[3 % kFaNp]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // dims 8 dv + 2e (low halves) and + 2e + 1 (high halves) of positions 0..3
      uint2 lo, hi;
      if constexpr (F16) {
        const float a0 = __uint_as_float(v0[e] << 16), a1 = __uint_as_float(v1[e] << 16);
        const float a2 = __uint_as_float(v2[e] << 16), a3 = __uint_as_float(v3[e] << 16);
        const float b0 = __uint_as_float(v0[e] & 0xffff0000u), b1 = __uint_as_float(v1[e] & 0xffff0000u);
        const float b2 = __uint_as_float(v2[e] & 0xffff0000u), b3 = __uint_as_float(v3[e] & 0xffff0000u);
        lo = make_uint2(pack_f16x2(a0, a1), pack_f16x2(a2, a3));
        hi = make_uint2(pack_f16x2(b0, b1), pack_f16x2(b2, b3));
        vmax = max3_abs(vmax, a0, a1);
        vmax = max3_abs(vmax, a2, a3);
        vmax = max3_abs(vmax, b0, b1);
        vmax = max3_abs(vmax, b2, b3);
      } else {
        lo = make_uint2(pack_low_halves(v0[e], v1[e]), pack_low_halves(v2[e], v3[e]));
        hi = make_uint2(pack_high_halves(v0[e], v1[e]), pack_high_halves(v2[e], v3[e]));
      }
      *reinterpret_cast<uint2*>(&s_vt[8 * dv + 2 * e][slot]) = lo;
      *reinterpret_cast<uint2*>(&s_vt[8 * dv + 2 * e + 1][slot]) = hi;
    }
    if constexpr (F16) {
      if (vmax > kFaF16VMax) s_big[buf] = b;
    }
    }
  };

  {
    // fp16 weights carry a factor 2^7 (the largest, 2^kLazyMax, becomes 2^15)
    // so that weights down to 2^-21 of the reference stay normal numbers; the
    // factor cancels in O / l
    constexpr float kPBias = F16 ? 7.0f : 0.0f;
    float m = -INFINITY, lsum = 0.0f;          // row n; lsum: this lane's positions only
    f32x16_t acc[4];                           // O^T tiles: dims 32 dt + 8 (v/4) + 4 hh + v%4
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][v] = 0.0f;

    int idk, idv;
    block_ids(0, idk, idv);
    fetch(0, idk, idv);
    if (nblk > 1) block_ids(1, idk, idv);
    if constexpr (F16) {
      // no block stamps yet (LDS keeps what an earlier workgroup left)
      if (tid < kFaBufs) s_big[tid] = -1;
      __syncthreads();
    }
    stage(0, 0);
    if (nblk > 1) {
      fetch(1, idk, idv);
      if (nblk > 2) block_ids(2, idk, idv);
    }
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
      const uint16_t(*s_k)[kFaKRow] = s_kb[blk & 1];
      const uint16_t(*s_vt)[kFaVRow] = s_vtb[blk & 1];
      const int cur = blk & 1;
      const int p0 = blk * kFaPos;
      if constexpr (F16) {
        if (__builtin_amdgcn_readfirstlane(s_big[cur]) == blk) return false;
      }
      // S^T tiles: sc[pt][v] = score of row n at position p0 + 32 pt + 8 (v/4) + 4 hh + v%4
      f32x16_t sc[2];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[pt][v] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8_t kop = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const uint4*>(&s_k[32 * pt + n][16 * ks + 8 * hh]));
          sc[pt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], sc[pt], 0, 0, 0);
        }
      }
      // B operands of the P.V steps: step st covers positions 16 st .. 16 st + 15;
      // this lane's k-slots 8 hh + 4 q + r are positions 16 st + 8 q + 4 hh + r,
      // i.e. its scores v = 8 (st % 2) .. + 7 of tile st / 2
      uint4 pb[4], pl[4];
      bool rescale;
      float alpha;
      auto softmax = [&](auto masked_tag) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        float bm = -INFINITY;
        if constexpr (kMasked) {
#pragma unroll
          for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              bm = p0 + 32 * pt + 8 * (v >> 2) + 4 * hh + (v & 3) <= pos_c ? fmaxf(bm, sc[pt][v]) : bm;
        } else {
          float b0 = -INFINITY, b1 = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            b0 = max3f(b0, sc[0][v], sc[0][v + 1]);
            b1 = max3f(b1, sc[1][v], sc[1][v + 1]);
          }
          bm = fmaxf(b0, b1);
        }
        bm = fmaxf(bm, xor_lanes<32>(bm));
        const float bms = bm == -INFINITY ? -INFINITY : bm * qs;
        const float mn = bms > m + kLazyMax ? bms : m;
        alpha = mn == m ? 1.0f : exp2_fast(m - mn);
        rescale = alpha != 1.0f;
        m = mn;
        const float mo = kPBias - mn;
        float p[2][16];
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            p[pt][v] = exp2_fast(fmaf(sc[pt][v], qs, mo));
            if constexpr (kMasked)
              p[pt][v] = p0 + 32 * pt + 8 * (v >> 2) + 4 * hh + (v & 3) <= pos_c ? p[pt][v] : 0.0f;
          }
        float ps = 0.0f;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float* f = &p[st >> 1][8 * (st & 1)];
          if constexpr (F16) {
            pb[st] = make_uint4(pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]),
                                pack_f16x2(f[4], f[5]), pack_f16x2(f[6], f[7]));
            // row sum of the weights as the matrix cores see them (fp16)
            const f16x2_t one2 = {1, 1};
            ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pb[st].x), one2, ps, false);
            ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pb[st].y), one2, ps, false);
            ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pb[st].z), one2, ps, false);
            ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pb[st].w), one2, ps, false);
          } else {
            uint32_t hb[4], lb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hb[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
              lb[e] = pack_bf16x2(f[2 * e] - __uint_as_float(hb[e] << 16),
                                  f[2 * e + 1] - __uint_as_float(hb[e] & 0xffff0000u));
              ps += f[2 * e] + f[2 * e + 1];
            }
            pb[st] = make_uint4(hb[0], hb[1], hb[2], hb[3]);
            pl[st] = make_uint4(lb[0], lb[1], lb[2], lb[3]);
          }
        }
        lsum = lsum * alpha + ps;
      };
      if (p0 + kFaPos <= vis_w)
        softmax(std::false_type{});
      else
        softmax(std::true_type{});
      if (__ballot(rescale) != 0) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
      }
      // O^T += V^T P^T: A = V^T (dim 32 dt + n, k-slots 8 hh ..), B = P^T (row n)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const uint4 vraw = *reinterpret_cast<const uint4*>(&s_vt[32 * dt + n][16 * st + 8 * hh]);
          if constexpr (F16) {
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, vraw),
                                                             __builtin_bit_cast(f16x8_t, pb[st]),
                                                             acc[dt], 0, 0, 0);
          } else {
            const bf16x8_t va = __builtin_bit_cast(bf16x8_t, vraw);
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, __builtin_bit_cast(bf16x8_t, pb[st]),
                                                              acc[dt], 0, 0, 0);
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, __builtin_bit_cast(bf16x8_t, pl[st]),
                                                              acc[dt], 0, 0, 0);
          }
        }
      if (blk + 1 < nblk) {
        // every wave finished block b - 1 before the barrier that ended it, so
        // its buffer ((b + 1) & 1) is free
        stage((blk + 1) & 1, blk + 1);
        if (blk + 2 < nblk) {
          fetch(blk + 2, idk, idv);
          if (blk + 3 < nblk) block_ids(blk + 3, idk, idv);
        }
      }
      __syncthreads();
    }
    // out[row n] = O[row n] / l; lane holds dims 32 dt + 8 gq + 4 hh + (0..3)
    const float l = lsum + xor_lanes<32>(lsum);
    const int row = roww + n;
    if (row < rows) {
      const int t = row / G, h = row % G;
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) +
                      ((int64_t)(q0 + t) * a.num_q_heads + g * G + h) * D + 4 * hh;
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint32_t lo = (uint32_t)bf16_bits(acc[dt][4 * gq] * inv) |
                              ((uint32_t)bf16_bits(acc[dt][4 * gq + 1] * inv) << 16);
          const uint32_t hi = (uint32_t)bf16_bits(acc[dt][4 * gq + 2] * inv) |
                              ((uint32_t)bf16_bits(acc[dt][4 * gq + 3] * inv) << 16);
          *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * gq) = make_uint2(lo, hi);
        }
    }
  }
  return true;
}

// Ticket of the latest multi-token call whose fp16 walk gave up on a tile
// (tickets only grow; 0: none yet), one per device.
__device__ unsigned long long g_fa_exact_ticket;

// F16: the fast pass; a tile that meets a V value beyond +-kFaF16VMax writes
// nothing and raises the call's ticket. !F16: the exact pass, launched right
// after on the same stream; it walks every tile again, but only when the
// ticket shows that some fp16 tile of this call (or of a later one, which
// costs a redundant pass and nothing else) gave up.
template <int BS, int G, bool F16>
__global__ __launch_bounds__(kFaRows * 2, 2) void multi_query_fa(MqArgs a) {
  __shared__ __align__(16) uint16_t s_kb[kFaBufs][kFaPos][kFaKRow];
  __shared__ __align__(16) uint16_t s_vtb[kFaBufs][128][kFaVRow];
  __shared__ int s_big[kFaBufs];
  if constexpr (!F16) {
    if (__hip_atomic_load(&g_fa_exact_ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
        a.fa_ticket)
      return;
  }
  if (!multi_query_fa_tile<BS, G, F16>(a, s_kb, s_vtb, s_big) && threadIdx.x == 0)
    atomicMax(&g_fa_exact_ticket, a.fa_ticket);
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
using PartitionKernel = void (*)(DecodeArgs);
using PartitionKernelMq = void (*)(MqArgs);

template <typename T, int D, int BS>
static PartitionKernel pick_valu(int group) {
  switch (group) {
    case 1: return decode_partition_valu<T, D, BS, 1, kDecodeWaves>;
    case 2: return decode_partition_valu<T, D, BS, 2, kDecodeWaves>;
    case 4: return decode_partition_valu<T, D, BS, 4, kDecodeWaves>;
    case 8: return decode_partition_valu<T, D, BS, 8, kDecodeWaves>;
    default: return nullptr;
  }
}

template <typename T>
static PartitionKernel pick_valu_t(int d, int bs, int group) {
  if (d == 64 && bs == 16) return pick_valu<T, 64, 16>(group);
  if (d == 64 && bs == 32) return pick_valu<T, 64, 32>(group);
  if (d == 128 && bs == 16) return pick_valu<T, 128, 16>(group);
  if (d == 128 && bs == 32) return pick_valu<T, 128, 32>(group);
  return nullptr;
}

template <int BS, bool F8, int POL, int NW>
static PartitionKernel pick_mfma_nw(int group) {
  switch (group) {
    case 1: return decode_partition_mfma<BS, 1, NW, F8, false, POL>;
    case 2: return decode_partition_mfma<BS, 2, NW, F8, false, POL>;
    case 4: return decode_partition_mfma<BS, 4, NW, F8, false, POL>;
    default: return nullptr;
  }
}

// Waves per workgroup of the matrix-core kernel for a shape whose full grid
// (sequences x KV heads x partitions) has `groups` workgroups:
// kMfmaDecodeWaves on grids that fill the chip several times over,
// kDecodeWaves on small batches, where a unit's latency (more chunks per
// wave) matters more than the end of the grid.
constexpr int64_t kMfmaNarrowMinGroups = 1024;
static int mfma_waves(int64_t groups) {
  return groups >= kMfmaNarrowMinGroups ? kMfmaDecodeWaves : kDecodeWaves;
}

template <int BS, bool F8, int POL>
static PartitionKernel pick_mfma_pol(int group, int waves) {
  return waves == kMfmaDecodeWaves ? pick_mfma_nw<BS, F8, POL, kMfmaDecodeWaves>(group)
                                   : pick_mfma_nw<BS, F8, POL, kDecodeWaves>(group);
}

template <int BS, bool F8>
static PartitionKernel pick_mfma(const DecodeKey& k, int waves) {
  return k.cached_kv ? pick_mfma_pol<BS, F8, kKvCached>(k.group, waves)
                     : pick_mfma_pol<BS, F8, kKvStream>(k.group, waves);
}

static PartitionKernel pick_partition(const DecodeKey& k, int waves = kDecodeWaves) {
  if (k.variant == 1) {
    if (k.kv_fp8) return nullptr;
    if (k.dtype == 0) return pick_valu_t<float>(k.head_dim, k.block_size, k.group);
    if (k.dtype == 1) return pick_valu_t<uint16_t>(k.head_dim, k.block_size, k.group);
    return nullptr;
  }
  if (k.variant == 2) {
    if (k.dtype != 1 || k.head_dim != 128) return nullptr;
    if (k.kv_fp8) {
      switch (k.block_size) {
        case 16: return pick_mfma<16, true>(k, waves);
        case 32: return pick_mfma<32, true>(k, waves);
        case 64: return pick_mfma<64, true>(k, waves);
        case 128: return pick_mfma<128, true>(k, waves);
        default: return nullptr;
      }
    }
    switch (k.block_size) {
      case 8: return pick_mfma<8, false>(k, waves);
      case 16: return pick_mfma<16, false>(k, waves);
      case 32: return pick_mfma<32, false>(k, waves);
      case 64: return pick_mfma<64, false>(k, waves);
      case 128: return pick_mfma<128, false>(k, waves);
      default: return nullptr;
    }
  }
  return nullptr;
}

bool decode_partition_supported(const DecodeKey& key) { return pick_partition(key) != nullptr; }

hipError_t launch_decode_partition(const DecodeKey& key, const DecodeArgs& args,
                                   hipStream_t stream) {
  const int64_t groups = (int64_t)args.num_kv_heads *
                        (args.plan ? (int64_t)args.num_units
                                   : (int64_t)args.num_seqs * args.max_parts);
  // the wave count follows the shape's full grid, so that a planned call
  // runs the same kernel as the unplanned one (bit-identical results)
  // (the shared-prefix walks run inside launch_shared_prefix_decode)
  if (args.pos_start) return hipErrorInvalidValue;
  const bool mfma = key.variant == 2;
  const int waves =
      mfma ? mfma_waves((int64_t)args.num_kv_heads * args.num_seqs * args.max_parts)
           : kDecodeWaves;
  PartitionKernel kern = pick_partition(key, waves);
  if (!kern) return hipErrorInvalidValue;
  if (groups <= 0) return hipSuccess;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)groups), dim3(waves * 64), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_decode_reduce(int dtype, int head_dim, const DecodeArgs& args,
                                hipStream_t stream) {
  if (args.max_parts <= 1 && !args.pos_start) return hipSuccess;
  const int64_t pairs = (int64_t)args.num_seqs * args.num_q_heads;
  if (pairs <= 0) return hipSuccess;
  if (pairs > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t groups = (pairs + kReduceWaves - 1) / kReduceWaves;
  PartitionKernel kern = nullptr;
  if (dtype == 0 && head_dim == 64) kern = decode_reduce<float, 64>;
  if (dtype == 0 && head_dim == 128) kern = decode_reduce<float, 128>;
  if (dtype == 1 && head_dim == 64) kern = decode_reduce<uint16_t, 64>;
  if (dtype == 1 && head_dim == 128) kern = decode_reduce<uint16_t, 128>;
  if (args.pos_start) kern = dtype == 1 && head_dim == 128 ? decode_reduce<uint16_t, 128, true> : nullptr;
  if (!kern) return hipErrorInvalidValue;
  // the shared-prefix decode's slots: prefix pass and walks
  const int64_t slots = args.pos_start ? (int64_t)args.slot_stride : args.max_parts;
  if (dtype == 1 && head_dim == 128 && args.num_q_heads == 4 * args.num_kv_heads &&
      slots <= kReduceFast) {
    // one wave per (sequence, KV head), every partition in one batch
    const int64_t units = (int64_t)args.num_seqs * args.num_kv_heads;
    hipLaunchKernelGGL(args.pos_start ? decode_reduce_g4<true> : decode_reduce_g4<false>,
                       dim3((unsigned)((units + kReduceWaves - 1) / kReduceWaves)),
                       dim3(kReduceWaves * 64), 0, stream, args);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)groups), dim3(kReduceWaves * 64), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const CacheArgs& args, hipStream_t stream) {
  const int64_t total = (int64_t)args.num_tokens * args.num_kv_heads * args.row_chunks;
  if (total <= 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(256), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_e4m3(const CacheArgs8& args, hipStream_t stream) {
  const int64_t total = (int64_t)args.num_tokens * args.num_kv_heads * args.row_groups;
  if (total <= 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reshape_and_cache_e4m3_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     args);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyArgs& args, hipStream_t stream) {
  if (args.num_pairs <= 0) return hipSuccess;
  const int64_t per_wg = 256 * 4;  // 16-byte chunks per workgroup sweep
  int64_t gy = (args.block_chunks + per_wg - 1) / per_wg;
  if (gy < 1) gy = 1;
  if (gy > 1024) gy = 1024;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)args.num_pairs, (unsigned)gy, 2),
                     dim3(256), 0, stream, args);
  return hipGetLastError();
}

bool multi_query_supported(int dtype, int head_dim, int block_size, int group) {
  return dtype == 1 && head_dim == 128 && (block_size == 16 || block_size == 32 ||
                                           block_size == 64 || block_size == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

template <int BS>
static PartitionKernelMq pick_mq(int group) {
  switch (group) {
    case 1: return multi_query_mfma<BS, 1>;
    case 2: return multi_query_mfma<BS, 2>;
    case 4: return multi_query_mfma<BS, 4>;
    case 8: return multi_query_mfma<BS, 8>;
    case 16: return multi_query_mfma<BS, 16>;
    default: return nullptr;
  }
}

bool multi_query_tiled(int group, int max_query_len);

template <int BS, bool F16>
static PartitionKernelMq pick_fa(int group) {
  switch (group) {
    case 1: return multi_query_fa<BS, 1, F16>;
    case 2: return multi_query_fa<BS, 2, F16>;
    case 4: return multi_query_fa<BS, 4, F16>;
    case 8: return multi_query_fa<BS, 8, F16>;
    case 16: return multi_query_fa<BS, 16, F16>;
    default: return nullptr;
  }
}

// process-wide source of the tickets of multi-token calls on the tiled path
static std::atomic<unsigned long long> g_fa_tickets{0};

hipError_t launch_multi_query(int block_size, int group, const MqArgs& args, hipStream_t stream) {
  if (multi_query_tiled(group, args.max_query_len)) {
    // many rows per (sequence, KV head): workgroup tiles sharing staged K/V
    PartitionKernelMq kern = nullptr, exact = nullptr;
    switch (block_size) {
      case 16: kern = pick_fa<16, true>(group); exact = pick_fa<16, false>(group); break;
      case 32: kern = pick_fa<32, true>(group); exact = pick_fa<32, false>(group); break;
      case 64: kern = pick_fa<64, true>(group); exact = pick_fa<64, false>(group); break;
      case 128: kern = pick_fa<128, true>(group); exact = pick_fa<128, false>(group); break;
      default: break;
    }
    if (!kern || !exact) return hipErrorInvalidValue;
    const int64_t tiles = ((int64_t)args.max_query_len * group + kFaRows - 1) / kFaRows;
    const int64_t pairs = (int64_t)args.num_seqs * args.num_kv_heads;
    if (pairs <= 0) return hipSuccess;
    const int64_t gx = 8 * tiles * ((pairs + 7) / 8);
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    MqArgs a = args;
    a.fa_ticket = ++g_fa_tickets;
    hipLaunchKernelGGL(kern, dim3((unsigned)gx), dim3(64 * kFaWaves), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(exact, dim3((unsigned)gx), dim3(64 * kFaWaves), 0, stream, a);
    return hipGetLastError();
  }
  hipError_t e = launch_multi_query_tiles(block_size, group, args, stream);
  if (e != hipSuccess || args.max_parts == 1) return e;
  return launch_multi_query_reduce(group, args, stream);
}

hipError_t launch_multi_query_tiles(int block_size, int group, const MqArgs& args,
                                   hipStream_t stream) {
  PartitionKernelMq kern = nullptr;
  switch (block_size) {
    case 16: kern = pick_mq<16>(group); break;
    case 32: kern = pick_mq<32>(group); break;
    case 64: kern = pick_mq<64>(group); break;
    case 128: kern = pick_mq<128>(group); break;
    default: break;
  }
  if (!kern) return hipErrorInvalidValue;
  if (args.max_parts < 1 || (args.max_parts > 1 && args.part_tokens <= 0))
    return hipErrorInvalidValue;
  const int64_t tiles = ((int64_t)args.max_query_len * group + 15) / 16;
  // a work plan (decode mode): one wave per listed unit, sequences from the plan
  const int64_t gx = args.plan ? ((int64_t)args.num_units + kMqWaves - 1) / kMqWaves
                               : (tiles * args.max_parts + kMqWaves - 1) / kMqWaves;
  const int64_t gz = args.plan ? 1 : args.num_seqs;
  if (gx <= 0 || args.num_seqs <= 0) return hipSuccess;
  if (gx > 0x7fffffff || args.num_kv_heads > 65535 || args.num_seqs > 65535)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)args.num_kv_heads, (unsigned)gz),
                     dim3(kMqWaves * 64), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_multi_query_reduce(int group, const MqArgs& args, hipStream_t stream) {
  // (shared-prefix decode always merges: its passes only leave partials)
  if (args.max_parts <= 1 && args.mode != 3) return hipSuccess;
  if (args.num_seqs <= 0 || args.num_seqs > 65535) return args.num_seqs <= 0 ? hipSuccess
                                                                              : hipErrorInvalidValue;
  PartitionKernelMq red = nullptr;
  switch (group) {
    case 1: red = multi_query_reduce<1>; break;
    case 2: red = multi_query_reduce<2>; break;
    case 4: red = multi_query_reduce<4>; break;
    case 8: red = multi_query_reduce<8>; break;
    case 16: red = multi_query_reduce<16>; break;
    default: return hipErrorInvalidValue;
  }
  const int64_t rx = ((int64_t)args.max_query_len * args.num_q_heads + kMqWaves - 1) / kMqWaves;
  if (rx > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(red, dim3((unsigned)rx, (unsigned)args.num_seqs), dim3(kMqWaves * 64), 0,
                     stream, args);
  return hipGetLastError();
}

template <int BS>
static void (*pick_cascade(int group))(CascadeArgs) {
  switch (group) {
    case 1: return shared_prefix_decode<BS, 1>;
    case 2: return shared_prefix_decode<BS, 2>;
    case 4: return shared_prefix_decode<BS, 4>;
    default: return nullptr;
  }
}

hipError_t launch_shared_prefix_decode(int block_size, int group, const MqArgs& pre,
                                       const DecodeArgs& walk, hipStream_t stream) {
  void (*kern)(CascadeArgs) = nullptr;
  switch (block_size) {
    case 16: kern = pick_cascade<16>(group); break;
    case 32: kern = pick_cascade<32>(group); break;
    case 64: kern = pick_cascade<64>(group); break;
    case 128: kern = pick_cascade<128>(group); break;
    default: break;
  }
  if (!kern || !walk.pos_start || pre.mode != 2) return hipErrorInvalidValue;
  CascadeArgs ca{};
  ca.pre = pre;
  ca.walk = walk;
  const int64_t tiles = ((int64_t)pre.max_query_len * group + 15) / 16;
  const int64_t pre_gx =
      pre.max_parts > 0 ? (tiles * pre.max_parts + kCascadeWaves - 1) / kCascadeWaves : 0;
  const int64_t n_prefix = pre_gx * pre.num_kv_heads * pre.num_seqs;
  // the walks: one workgroup per (unit, KV head) of a work plan, else the
  // full (sequence, partition, KV head) grid
  const int64_t n_walk = (int64_t)walk.num_kv_heads *
                         (walk.plan ? (int64_t)walk.num_units
                                    : (int64_t)walk.num_seqs * walk.max_parts);
  if (n_prefix + n_walk <= 0) return hipSuccess;
  if (n_prefix + n_walk > 0x7fffffff) return hipErrorInvalidValue;
  ca.n_prefix = (int32_t)n_prefix;
  ca.pre_gx = (int32_t)(pre_gx > 0 ? pre_gx : 1);
  hipLaunchKernelGGL(kern, dim3((unsigned)(n_prefix + n_walk)), dim3(kCascadeWaves * 64), 0, stream,
                     ca);
  return hipGetLastError();
}

bool multi_query_tiled(int group, int max_query_len) {
  return (int64_t)max_query_len * group >= kFaMinRows;
}

// Copy of the error word taken by take_errors_kernel.
__device__ uint32_t g_error_snapshot;

// Fetches and clears the error word in one atomic exchange, so that a bit
// raised by work still running elsewhere (another stream) stays set for the
// next read instead of being lost between a read and a separate clear.
__global__ void take_errors_kernel() {
  if (threadIdx.x == 0) g_error_snapshot = atomicExch(&g_error_word, 0u);
}

hipError_t read_and_clear_errors(uint32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(take_errors_kernel, dim3(1), dim3(64), 0, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t v = 0;
  e = hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_error_snapshot), sizeof(v), 0,
                               hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  *flags = v;
  return hipSuccess;
}

}  // namespace pa
