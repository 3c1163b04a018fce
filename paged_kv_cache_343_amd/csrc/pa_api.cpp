// C ABI of libpa: argument validation and kernel dispatch. Every check on a
// host-visible argument happens before anything is enqueued; on error the
// call returns a status and enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kDefaultPartitionTokens = 512;
// Contexts longer than this get automatic partitions of kLongPartitionTokens:
// every partition writes a partial output (HBM writes in the middle of the
// streaming K/V reads, which cost far more than their bytes), and a long
// context has many (a 32,768-position sequence: 64 of 512 positions).
constexpr int kLongContext = 8192;
constexpr int kLongPartitionTokens = 1024;
// pa_multi_query_split: one wave walks a partition for a whole 16-row tile,
// so partitions are longer than decode's (measured best on 4-token chunks)
constexpr int kDefaultMqPartitionTokens = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : 0; }

// Resolved layout of a decode call.
struct Plan {
  int part_tokens = 0;
  int max_parts = 0;
  int len_cap = 0;
  int group = 0;
  size_t ml_bytes = 0;    // partial (max, sum) region
  size_t o_bytes = 0;     // partial output region
  bool part_half = false; // partial outputs in bf16
  bool mq_route = false;  // runs on the multi-token per-tile kernel
  pa::DecodeKey key{};
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// pa_decode_shape_t.variant: kernel choice in the low byte, hint flags above.
constexpr int kVariantMask = 0xff;

int auto_variant(const pa_decode_shape_t& s, int group) {
  if (s.dtype == PA_BF16 && s.head_dim == 128 &&
      (group == 1 || group == 2 || group == 4 || group == 8 || group == 16))
    return PA_VARIANT_MFMA;
  return PA_VARIANT_VALU;
}

// Matrix-core decode with 8 or 16 query heads per KV head runs on the
// multi-token per-tile kernel (one 16-row tile = the whole group, both
// products on the matrix cores) in its one-token-per-sequence mode.
bool decode_on_multi_query(const pa_decode_shape_t& s, int group, int variant, bool kv_fp8) {
  return !kv_fp8 && variant == PA_VARIANT_MFMA && (group == 8 || group == 16) &&
         pa::multi_query_supported(s.dtype, s.head_dim, s.block_size, group);
}

pa_status_t make_plan(const pa_decode_shape_t* s, Plan* plan, bool kv_fp8 = false) {
  if (!s) return PA_EINVAL;
  if (s->num_seqs < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->num_blocks <= 0 ||
      s->max_blocks_per_seq <= 0 || s->max_seq_len < 0 || s->block_size <= 0 ||
      s->head_dim <= 0)
    return PA_EINVAL;
  if (s->num_q_heads % s->num_kv_heads != 0) return PA_EINVAL;
  if (elem_bytes(s->dtype) == 0) return PA_EINVAL;
  if ((s->head_dim * elem_bytes(s->dtype)) % 16 != 0) return PA_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return PA_EUNSUPPORTED;
  if (s->block_size != 8 && s->block_size != 16 && s->block_size != 32 && s->block_size != 64 &&
      s->block_size != 128)
    return PA_EUNSUPPORTED;
  const int group = s->num_q_heads / s->num_kv_heads;
  if (s->variant & ~(kVariantMask | PA_DECODE_SHARED_KV | PA_DECODE_HALF_PARTIALS))
    return PA_EINVAL;
  const int base = s->variant & kVariantMask;
  int variant = base == PA_VARIANT_AUTO ? auto_variant(*s, group) : base;
  if (variant != PA_VARIANT_VALU && variant != PA_VARIANT_MFMA) return PA_EINVAL;
  plan->mq_route = decode_on_multi_query(*s, group, variant, kv_fp8);
  int pt = s->partition_tokens;
  // automatic length: 512 positions; 1024 on the per-tile kernel (one wave
  // walks a partition for the whole group; measured best at group 8), for
  // 8-bit pools (the same bytes per workgroup as 512 bf16 positions) and for
  // contexts beyond kLongContext (fewer partial outputs)
  if (pt == 0)
    pt = plan->mq_route || kv_fp8 ? kDefaultMqPartitionTokens
         : s->max_seq_len > kLongContext ? kLongPartitionTokens
                                         : kDefaultPartitionTokens;
  if (pt == -1) {
    // one partition per sequence
    pt = s->max_seq_len > 0 ? (int)round_up((size_t)s->max_seq_len, (size_t)s->block_size)
                            : s->block_size;
  }
  if (pt <= 0 || pt % s->block_size != 0) return PA_EINVAL;
  plan->part_tokens = pt;
  plan->max_parts = s->max_seq_len == 0 ? 1 : (s->max_seq_len + pt - 1) / pt;
  const int64_t table_cap = (int64_t)s->max_blocks_per_seq * s->block_size;
  plan->len_cap = (int)(table_cap < s->max_seq_len ? table_cap : s->max_seq_len);
  plan->group = group;
  plan->key = pa::DecodeKey{s->dtype, s->head_dim, s->block_size, group, variant, kv_fp8,
                            (s->variant & PA_DECODE_SHARED_KV) != 0};
  if (!plan->mq_route && !pa::decode_partition_supported(plan->key)) return PA_EUNSUPPORTED;
  if (group * 2 > pa::kMlRecord) return PA_EUNSUPPORTED;
  const size_t rows = (size_t)s->num_seqs * s->num_q_heads * plan->max_parts;
  const size_t recs = (size_t)s->num_seqs * s->num_kv_heads * plan->max_parts;
  if (plan->max_parts > 1) {
    plan->ml_bytes = round_up(recs * pa::kMlRecord * sizeof(float), 256);
    // bf16 partials only on request, for full-length partitions of the
    // decode kernels (the per-tile multi-token kernel keeps fp32)
    plan->part_half = (s->variant & PA_DECODE_HALF_PARTIALS) && s->dtype == PA_BF16 &&
                      pt >= pa::kHalfPartialMinTokens && !plan->mq_route;
    plan->o_bytes = round_up(rows * (size_t)s->head_dim * 4, 256);
  }
  return PA_OK;
}

pa_status_t fill_args(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, float scale, void* out,
                      const pa_decode_shape_t* s, const Plan& plan, void* workspace,
                      size_t workspace_bytes, pa::DecodeArgs* a) {
  if (s->num_seqs > 0 && (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out))
    return PA_EINVAL;
  if (s->num_seqs > 0 &&
      (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)))
    return PA_EINVAL;
  if (!std::isfinite(scale)) return PA_EINVAL;
  const size_t need = plan.ml_bytes + plan.o_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PA_EWORKSPACE;
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->block_tables = block_tables;
  a->seq_lens = seq_lens;
  a->out = out;
  a->part_ml = need > 0 ? static_cast<float*>(workspace) : nullptr;
  a->part_o = need > 0 ? static_cast<void*>(static_cast<char*>(workspace) + plan.ml_bytes)
                       : nullptr;
  a->qscale = scale * 1.4426950408889634f;  // log2(e): scores kept in log2 units
  a->out_scale = 1.0f;
  a->part_half = plan.part_half ? 1 : 0;
  a->num_seqs = s->num_seqs;
  a->num_q_heads = s->num_q_heads;
  a->num_kv_heads = s->num_kv_heads;
  a->num_blocks = s->num_blocks;
  a->max_blocks = s->max_blocks_per_seq;
  a->max_seq_len = s->max_seq_len;
  a->len_cap = plan.len_cap;
  a->part_tokens = plan.part_tokens;
  a->max_parts = plan.max_parts;
  return PA_OK;
}

// The HIP error behind the calling thread's most recent PA_EHIP.
thread_local hipError_t g_last_hip_error = hipSuccess;

pa_status_t from_hip(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  g_last_hip_error = e;
  return PA_EHIP;
}

}  // namespace

extern "C" {

size_t pa_decode_workspace_bytes(const pa_decode_shape_t* shape) {
  Plan plan;
  if (make_plan(shape, &plan) != PA_OK) return 0;
  return plan.ml_bytes + plan.o_bytes;
}

// Decode on the multi-token per-tile kernel (8 or 16 query heads per KV head
// on the matrix cores), one token per sequence, in the same workspace
// regions: per (sequence, query head, partition) the (max, exp-sum) pair
// (within the statistics records' space) and the partial output in the
// decode layout.
static pa::MqArgs decode_mq_args(const pa::DecodeArgs& a, const pa_decode_shape_t& shape,
                                 const Plan& plan) {
  pa::MqArgs m{};
  m.q = a.q;
  m.k_pool = a.k_pool;
  m.v_pool = a.v_pool;
  m.block_tables = a.block_tables;
  m.seq_lens = a.seq_lens;
  m.out = a.out;
  m.qscale = a.qscale;
  m.num_seqs = a.num_seqs;
  m.num_q_heads = a.num_q_heads;
  m.num_kv_heads = a.num_kv_heads;
  m.num_blocks = a.num_blocks;
  m.max_blocks = a.max_blocks;
  m.len_cap = a.len_cap;
  m.max_query_len = 1;
  m.num_tokens = a.num_seqs;
  m.block_size = shape.block_size;
  m.decode_mode = 1;
  m.max_parts = plan.max_parts;
  m.part_tokens = plan.max_parts > 1 ? plan.part_tokens : 0;
  m.part_ml = a.part_ml;
  m.part_o = a.part_o;
  m.part_half = a.part_half;
  m.plan = a.plan;
  m.num_units = a.num_units;
  return m;
}

static pa_status_t decode_impl(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, const int32_t* seq_lens, float scale,
                               void* out, const pa_decode_shape_t* shape, void* workspace,
                               size_t workspace_bytes, void* stream, bool do_partition,
                               bool do_reduce, const float* fp8_scales = nullptr,
                               const int32_t* work_plan = nullptr, int32_t num_units = -1) {
  Plan plan;
  if (fp8_scales && shape &&
      (shape->dtype != PA_BF16 || (shape->variant & kVariantMask) == PA_VARIANT_VALU))
    return PA_EUNSUPPORTED;
  pa_decode_shape_t s8{};
  if (fp8_scales) {           // the 8-bit kernel is a matrix-core variant
    s8 = *shape;
    s8.variant = PA_VARIANT_MFMA | (shape->variant & ~kVariantMask);
    shape = &s8;
  }
  pa_status_t st = make_plan(shape, &plan, fp8_scales != nullptr);
  if (st != PA_OK) return st;
  pa::DecodeArgs a{};
  st = fill_args(q, k_pool, v_pool, block_tables, seq_lens, scale, out, shape, plan, workspace,
                 workspace_bytes, &a);
  if (st != PA_OK) return st;
  if (fp8_scales) {
    if (!std::isfinite(fp8_scales[0]) || !std::isfinite(fp8_scales[1]) || fp8_scales[0] <= 0.0f ||
        fp8_scales[1] <= 0.0f)
      return PA_EINVAL;
    a.qscale *= fp8_scales[0];
    a.out_scale = fp8_scales[1];
  }
  if (num_units >= 0) {
    // a work plan from pa_decode_plan
    if ((int64_t)num_units > (int64_t)shape->num_seqs * plan.max_parts) return PA_EINVAL;
    if (num_units > 0 && (!work_plan || !aligned16(work_plan)))
      return PA_EINVAL;
    a.plan = work_plan;
    a.num_units = num_units;
    if (num_units == 0) do_partition = false;   // nothing to compute or zero
  }
  if (shape->num_seqs == 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.mq_route) {
    const pa::MqArgs m = decode_mq_args(a, *shape, plan);
    if (do_partition) {
      st = from_hip(pa::launch_multi_query_tiles(shape->block_size, plan.group, m, s));
      if (st != PA_OK) return st;
    }
    if (do_reduce) st = from_hip(pa::launch_multi_query_reduce(plan.group, m, s));
    return st;
  }
  if (do_partition) {
    st = from_hip(pa::launch_decode_partition(plan.key, a, s));
    if (st != PA_OK) return st;
  }
  if (do_reduce) st = from_hip(pa::launch_decode_reduce(shape->dtype, shape->head_dim, a, s));
  return st;
}

// A work plan argument: null = the full grid (num_units must be 0), else a
// device array of num_units >= 0 entries from pa_decode_plan.
static bool plan_args_ok(const int32_t* work_plan, int32_t num_units) {
  return work_plan ? num_units >= 0 : num_units == 0;
}

pa_status_t pa_decode(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, float scale,
                      void* out, const pa_decode_shape_t* shape, const int32_t* work_plan,
                      int32_t num_units, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan_args_ok(work_plan, num_units)) return PA_EINVAL;
  return decode_impl(q, k_pool, v_pool, block_tables, seq_lens, scale, out, shape, workspace,
                     workspace_bytes, stream, true, true, nullptr, work_plan,
                     work_plan ? num_units : -1);
}

pa_status_t pa_decode_partition(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                float scale, void* out, const pa_decode_shape_t* shape,
                                const int32_t* work_plan, int32_t num_units, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!plan_args_ok(work_plan, num_units)) return PA_EINVAL;
  return decode_impl(q, k_pool, v_pool, block_tables, seq_lens, scale, out, shape, workspace,
                     workspace_bytes, stream, true, false, nullptr, work_plan,
                     work_plan ? num_units : -1);
}

int64_t pa_decode_plan_capacity(const pa_decode_shape_t* shape) {
  Plan plan;
  if (make_plan(shape, &plan) != PA_OK) return 0;
  return (int64_t)shape->num_seqs * plan.max_parts;
}

pa_status_t pa_decode_plan(const pa_decode_shape_t* shape, const int32_t* seq_lens,
                           const int32_t* walk_start, int32_t* work_plan, int64_t capacity,
                           int32_t* num_units) {
  Plan plan;
  pa_status_t st = make_plan(shape, &plan);
  if (st != PA_OK) return st;
  if (!num_units || (shape->num_seqs > 0 && (!seq_lens || !work_plan))) return PA_EINVAL;
  const int pt = plan.part_tokens;
  // positions [start, len) of each sequence are split into partitions
  auto start_of = [&](int32_t i) { return walk_start ? walk_start[i] : 0; };
  for (int32_t i = 0; i < shape->num_seqs; ++i) {
    const int32_t len = seq_lens[i], st0 = start_of(i);
    if (len < 0 || len > plan.len_cap || st0 < 0 || st0 > len) return PA_EINVAL;
  }
  // Units with a full partition come first, in (sequence, partition) order;
  // then each sequence's last, shorter partition (and the zero-output unit
  // of an empty sequence), longest first, so that the grid ends on the
  // shortest work. A walk that starts at its sequence's end has no unit.
  int64_t n = 0;
  for (int32_t i = 0; i < shape->num_seqs; ++i) {
    const int32_t len = seq_lens[i], st0 = start_of(i);
    const int full = (len - st0) / pt;
    if (n + full > capacity) return PA_EINVAL;
    for (int j = 0; j < full; ++j) {
      int32_t* e = work_plan + 4 * n++;
      e[0] = i;
      e[1] = j;
      e[2] = len;
      e[3] = st0;
    }
  }
  // tail units: longest first, sequence order among equals
  std::vector<int32_t> tail;   // sequences with a shorter last partition (or none at all)
  for (int32_t i = 0; i < shape->num_seqs; ++i) {
    const int32_t rest = seq_lens[i] - start_of(i);
    if (seq_lens[i] == 0 || rest % pt != 0) tail.push_back(i);
  }
  const int64_t tails = (int64_t)tail.size();
  if (n + tails > capacity) return PA_EINVAL;
  auto put = [&](int64_t u, int32_t i) {
    int32_t* e = work_plan + 4 * u;
    e[0] = i;
    e[1] = (seq_lens[i] - start_of(i)) / pt;
    e[2] = seq_lens[i];
    e[3] = start_of(i);
  };
  auto rem = [&](int32_t i) { return (seq_lens[i] - start_of(i)) % pt; };
  if (pt <= 65536) {
    // counting sort on the last partition's length
    std::vector<int32_t> start(pt + 2, 0);
    for (int32_t i : tail) ++start[rem(i)];
    int32_t acc = 0;
    for (int c = pt; c >= 0; --c) {
      const int32_t k = start[c];
      start[c] = acc;
      acc += k;
    }
    for (int32_t i : tail) put(n + start[rem(i)]++, i);
  } else {
    std::stable_sort(tail.begin(), tail.end(),
                     [&](int32_t x, int32_t y) { return rem(x) > rem(y); });
    for (int64_t k = 0; k < tails; ++k) put(n + k, tail[k]);
  }
  n += tails;
  if (n > INT32_MAX) return PA_EINVAL;
  *num_units = (int32_t)n;
  return PA_OK;
}

pa_status_t pa_decode_e4m3(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens, float scale,
                           float k_scale, float v_scale, void* out,
                           const pa_decode_shape_t* shape, const int32_t* work_plan,
                           int32_t num_units, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!plan_args_ok(work_plan, num_units)) return PA_EINVAL;
  if (work_plan && (!shape || shape->partition_tokens == 0)) return PA_EINVAL;
  const float sc[2] = {k_scale, v_scale};
  return decode_impl(q, k_pool, v_pool, block_tables, seq_lens, scale, out, shape, workspace,
                     workspace_bytes, stream, true, true, sc, work_plan,
                     work_plan ? num_units : -1);
}

pa_status_t pa_decode_partition_e4m3(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_tables, const int32_t* seq_lens,
                                     float scale, float k_scale, float v_scale, void* out,
                                     const pa_decode_shape_t* shape, const int32_t* work_plan,
                                     int32_t num_units, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!plan_args_ok(work_plan, num_units)) return PA_EINVAL;
  if (work_plan && (!shape || shape->partition_tokens == 0)) return PA_EINVAL;
  const float sc[2] = {k_scale, v_scale};
  return decode_impl(q, k_pool, v_pool, block_tables, seq_lens, scale, out, shape, workspace,
                     workspace_bytes, stream, true, false, sc, work_plan,
                     work_plan ? num_units : -1);
}

pa_status_t pa_decode_reduce(const int32_t* seq_lens, void* out, const pa_decode_shape_t* shape,
                             void* workspace, size_t workspace_bytes, void* stream) {
  Plan plan;
  pa_status_t st = make_plan(shape, &plan);
  if (st != PA_OK) return st;
  if (shape->num_seqs == 0 || plan.max_parts <= 1) return PA_OK;
  if (!seq_lens || !out || !aligned16(out)) return PA_EINVAL;
  const size_t need = plan.ml_bytes + plan.o_bytes;
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PA_EWORKSPACE;
  pa::DecodeArgs a{};
  a.seq_lens = seq_lens;
  a.out = out;
  a.part_ml = static_cast<float*>(workspace);
  a.part_o = static_cast<void*>(static_cast<char*>(workspace) + plan.ml_bytes);
  a.part_half = plan.part_half ? 1 : 0;
  a.num_seqs = shape->num_seqs;
  a.num_q_heads = shape->num_q_heads;
  a.num_kv_heads = shape->num_kv_heads;
  a.num_blocks = shape->num_blocks;
  a.max_blocks = shape->max_blocks_per_seq;
  a.max_seq_len = shape->max_seq_len;
  a.len_cap = plan.len_cap;
  a.part_tokens = plan.part_tokens;
  a.max_parts = plan.max_parts;
  if (plan.mq_route)   // the per-tile kernel's partials: its own merge
    return from_hip(pa::launch_multi_query_reduce(plan.group, decode_mq_args(a, *shape, plan),
                                                  static_cast<hipStream_t>(stream)));
  return from_hip(pa::launch_decode_reduce(shape->dtype, shape->head_dim, a,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// pa_decode_noalloc: pa_decode with its workspace in a file-scope device array
// ---------------------------------------------------------------------------
// Each GPU the library runs on holds its own copy of `scratch`, from the
// first call on that GPU until the process ends. In host code the name
// `scratch` is a host-side stand-in, not device memory: the kernels get the
// address hipGetSymbolAddress returns on the current device, resolved once
// per device and kept in g_scratch_addr.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's `scratch`.
pa_status_t scratch_address(void** addr) {
  int dev = -1;
  if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess) return from_hip(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return PA_EUNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return from_hip(e != hipSuccess ? e : hipErrorInvalidSymbol);
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return PA_OK;
}

}  // namespace

extern "C" pa_status_t pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                         const int32_t* block_tables, const int32_t* seq_lens,
                                         float scale, void* out, const pa_decode_shape_t* shape,
                                         void* stream) {
  Plan plan;
  pa_status_t st = make_plan(shape, &plan);
  if (st != PA_OK) return st;
  const size_t need = plan.ml_bytes + plan.o_bytes;
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_EWORKSPACE;
  // every partial the merge reads is written earlier in the same call, so
  // nothing in the array has to start at zero
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != PA_OK) return st;
  }
  return decode_impl(q, k_pool, v_pool, block_tables, seq_lens, scale, out, shape, ws, need,
                     stream, true, true);
}

namespace {

// Shared-prefix decode plan: partitions of the prefix pass, then of the
// per-sequence pass, in one partial array per (sequence, query head).
struct PrefixPlan {
  Plan base;              // the per-sequence walks (pa_decode's partitions)
  int pref_tokens = 0;    // partition length of the prefix pass
  int pref_parts = 0, suf_parts = 0;
  size_t ml_bytes = 0, o_bytes = 0;
};

pa_status_t prefix_plan(const pa_decode_shape_t* s, int32_t max_group_size,
                        int32_t max_prefix_len, PrefixPlan* pp) {
  if (!s || max_group_size <= 0 || max_prefix_len < 0) return PA_EINVAL;
  pa_decode_shape_t s2 = *s;
  s2.variant = PA_VARIANT_MFMA | (s->variant & PA_DECODE_HALF_PARTIALS);
  if (s2.partition_tokens == -1) return PA_EINVAL;
  pa_status_t st = make_plan(&s2, &pp->base);
  if (st != PA_OK) return st;
  const int group = s->num_q_heads / s->num_kv_heads;
  if (!pa::multi_query_supported(s->dtype, s->head_dim, s->block_size, group))
    return PA_EUNSUPPORTED;
  if (max_prefix_len % s->block_size != 0 || max_prefix_len > s->max_seq_len) return PA_EINVAL;
  if ((int64_t)max_group_size * group > (1 << 24)) return PA_EINVAL;
  // both passes use pa_decode's partitions: shorter prefix partitions would
  // spread the prefix pass over more waves but write more partial outputs
  // (the prefix pass runs beside the walks in one launch; 256-position
  // prefix partitions measured 95.5 vs 93.5 us on 64 x 4 samples of a
  // 1040-position prompt, 488 vs 475 us with 16 more 32,768-position
  // sequences)
  const int pt = pp->base.part_tokens;
  pp->pref_tokens = pt;
  pp->pref_parts = (max_prefix_len + pp->pref_tokens - 1) / pp->pref_tokens;
  pp->suf_parts = s->max_seq_len == 0 ? 1 : (s->max_seq_len + pt - 1) / pt;
  const size_t slots = (size_t)(pp->pref_parts + pp->suf_parts);
  // statistics in pa_decode's 128-byte records per (sequence, KV head, slot)
  // (the group-8/16 path keeps a pair per query row in the same space)
  pp->ml_bytes = round_up((size_t)s->num_seqs * s->num_kv_heads * slots * pa::kMlRecord *
                              sizeof(float), 256);
  pp->o_bytes = round_up((size_t)s->num_seqs * s->num_q_heads * slots * s->head_dim * 4, 256);
  // the decode kernel's own partitions keep bf16 partials on request (prefix
  // pass: fp32)
  pp->base.part_half = (s->variant & PA_DECODE_HALF_PARTIALS) && s->dtype == PA_BF16 &&
                       pt >= pa::kHalfPartialMinTokens && group <= 4;
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_decode_shared_prefix_workspace_bytes(const pa_decode_shape_t* shape,
                                               int32_t max_group_size, int32_t max_prefix_len) {
  PrefixPlan pp;
  if (prefix_plan(shape, max_group_size, max_prefix_len, &pp) != PA_OK) return 0;
  return pp.ml_bytes + pp.o_bytes;
}

pa_status_t pa_decode_shared_prefix(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    float scale, void* out, const pa_decode_shape_t* shape,
                                    int32_t num_groups, const int32_t* group_start,
                                    const int32_t* prefix_lens, int32_t max_group_size,
                                    int32_t max_prefix_len, const int32_t* work_plan,
                                    int32_t num_units, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  PrefixPlan pp;
  pa_status_t st = prefix_plan(shape, max_group_size, max_prefix_len, &pp);
  if (st != PA_OK) return st;
  if (!plan_args_ok(work_plan, num_units)) return PA_EINVAL;
  if (work_plan && ((int64_t)num_units > (int64_t)shape->num_seqs * pp.suf_parts ||
                    (num_units > 0 && !aligned16(work_plan))))
    return PA_EINVAL;
  if (num_groups < 0 || (num_groups > 0 && !group_start) || !prefix_lens) return PA_EINVAL;
  if (shape->num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out) return PA_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PA_EINVAL;
  if (!std::isfinite(scale)) return PA_EINVAL;
  const size_t need = pp.ml_bytes + pp.o_bytes;
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PA_EWORKSPACE;
  if (num_groups > 65535 || shape->num_seqs > 65535) return PA_EUNSUPPORTED;
  const int group = shape->num_q_heads / shape->num_kv_heads;
  pa::MqArgs m{};
  m.q = q;
  m.k_pool = k_pool;
  m.v_pool = v_pool;
  m.block_tables = block_tables;
  m.seq_lens = seq_lens;
  m.out = out;
  m.qscale = scale * 1.4426950408889634f;
  m.num_seqs = shape->num_seqs;
  m.num_q_heads = shape->num_q_heads;
  m.num_kv_heads = shape->num_kv_heads;
  m.num_blocks = shape->num_blocks;
  m.max_blocks = shape->max_blocks_per_seq;
  m.len_cap = pp.base.len_cap;
  m.num_tokens = shape->num_seqs;
  m.block_size = shape->block_size;
  m.part_tokens = pp.base.part_tokens;
  m.prefix_part_tokens = pp.pref_tokens;
  m.max_parts = pp.pref_parts + pp.suf_parts;
  m.part_ml = static_cast<float*>(workspace);
  m.part_o = static_cast<char*>(workspace) + pp.ml_bytes;
  m.part_half = pp.base.part_half ? 1 : 0;
  m.group_start = group_start;
  m.prefix_lens = prefix_lens;
  m.suffix_slot0 = pp.pref_parts;
  m.max_prefix = max_prefix_len;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // 1. per group: the shared prefix, the group's sequences as query rows
  m.slot_stride = pp.pref_parts + pp.suf_parts;
  m.part_half = 0;
  const bool decode_kernel = group <= 4;   // the walks on pa_decode's kernel
  if (work_plan && !decode_kernel) return PA_EINVAL;   // plans serve those walks only
  pa::MqArgs m2 = m;
  m2.mode = 2;
  m2.part_tokens = pp.pref_tokens;
  m2.num_seqs = num_groups;       // the grid runs over groups
  m2.max_query_len = max_group_size;
  m2.max_parts = num_groups > 0 ? pp.pref_parts : 0;
  m2.ml_records = decode_kernel ? 1 : 0;
  if (!decode_kernel && m2.max_parts > 0) {
    st = from_hip(pa::launch_multi_query_tiles(shape->block_size, group, m2, s));
    if (st != PA_OK) return st;
  }
  if (decode_kernel) {
    // 1 + 2. the prefix pass and the walks after the prefix (pa_decode's
    //    kernel, per (sequence, KV head, partition)) in one launch; 3. the
    //    decode reduce merges both passes' slots
    pa::DecodeArgs a{};
    st = fill_args(q, k_pool, v_pool, block_tables, seq_lens, scale, out, shape, pp.base,
                   workspace, workspace_bytes, &a);
    if (st != PA_OK) return st;
    a.part_ml = static_cast<float*>(workspace);
    a.part_o = static_cast<char*>(workspace) + pp.ml_bytes;
    a.part_tokens = pp.base.part_tokens;
    a.max_parts = pp.suf_parts;
    a.part_half = pp.base.part_half ? 1 : 0;
    a.pos_start = prefix_lens;
    a.prefix_part_tokens = pp.pref_tokens;
    a.slot0 = pp.pref_parts;
    a.slot_stride = pp.pref_parts + pp.suf_parts;
    a.max_prefix = max_prefix_len;
    a.block_size = shape->block_size;
    if (work_plan) {
      a.plan = work_plan;
      a.num_units = num_units;
    }
    st = from_hip(pa::launch_shared_prefix_decode(shape->block_size, group, m2, a, s));
    if (st != PA_OK) return st;
    return from_hip(pa::launch_decode_reduce(shape->dtype, shape->head_dim, a, s));
  }
  // 2. per sequence: the positions after its prefix
  pa::MqArgs m3 = m;
  m3.mode = 3;
  m3.max_query_len = 1;
  m3.max_parts = pp.suf_parts;
  st = from_hip(pa::launch_multi_query_tiles(shape->block_size, group, m3, s));
  if (st != PA_OK) return st;
  // 3. merge both passes' partials
  m3.max_parts = m.slot_stride;
  return from_hip(pa::launch_multi_query_reduce(group, m3, s));
}

}  // extern "C"

namespace {

// Validates a multi-query shape (not its pointers).
pa_status_t check_mq_shape(const pa_multi_query_shape_t* s) {
  if (!s) return PA_EINVAL;
  if (s->num_seqs < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->num_blocks <= 0 ||
      s->max_blocks_per_seq <= 0 || s->max_seq_len < 0 || s->max_query_len < 0 ||
      s->num_tokens < 0 || s->block_size <= 0 || s->head_dim <= 0)
    return PA_EINVAL;
  if (s->num_q_heads % s->num_kv_heads != 0 || elem_bytes(s->dtype) == 0) return PA_EINVAL;
  if (!pa::multi_query_supported(s->dtype, s->head_dim, s->block_size,
                                 s->num_q_heads / s->num_kv_heads))
    return PA_EUNSUPPORTED;
  return PA_OK;
}

struct MqSplit {
  int part_tokens = 0;   // 0: no split
  int max_parts = 1;
  bool part_half = false;
  size_t ml_bytes = 0, o_bytes = 0;
};

// Partition plan of pa_multi_query_split (partition_tokens 0 = the default).
pa_status_t mq_split_plan(const pa_multi_query_shape_t* s, int32_t partition_tokens,
                          MqSplit* sp) {
  pa_status_t st = check_mq_shape(s);
  if (st != PA_OK) return st;
  const int pt = partition_tokens == 0 ? kDefaultMqPartitionTokens : partition_tokens;
  if (pt <= 0 || pt % 16 != 0) return PA_EINVAL;
  sp->part_tokens = pt;
  sp->max_parts = s->max_seq_len == 0 ? 1 : (s->max_seq_len + pt - 1) / pt;
  if (pa::multi_query_tiled(s->num_q_heads / s->num_kv_heads, s->max_query_len))
    sp->max_parts = 1;   // the tiled kernel never splits
  if (sp->max_parts > 1) {
    const size_t rows = (size_t)s->num_tokens * s->num_q_heads * sp->max_parts;
    sp->part_half = false;
    sp->ml_bytes = round_up(rows * 2 * sizeof(float), 256);
    sp->o_bytes = round_up(rows * (size_t)s->head_dim * 4, 256);
  }
  return PA_OK;
}

pa_status_t multi_query_impl(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             const int32_t* query_start, float scale, void* out,
                             const pa_multi_query_shape_t* s, const MqSplit& sp,
                             void* workspace, void* stream) {
  const int group = s->num_q_heads / s->num_kv_heads;
  if (!std::isfinite(scale)) return PA_EINVAL;
  if (s->num_seqs == 0 || s->num_tokens == 0 || s->max_query_len == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !query_start || !out)
    return PA_EINVAL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PA_EINVAL;
  pa::MqArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start = query_start;
  a.out = out;
  a.qscale = scale * 1.4426950408889634f;
  a.num_seqs = s->num_seqs;
  a.num_q_heads = s->num_q_heads;
  a.num_kv_heads = s->num_kv_heads;
  a.num_blocks = s->num_blocks;
  a.max_blocks = s->max_blocks_per_seq;
  const int64_t table_cap = (int64_t)s->max_blocks_per_seq * s->block_size;
  a.len_cap = (int)(table_cap < s->max_seq_len ? table_cap : s->max_seq_len);
  a.max_query_len = s->max_query_len;
  a.num_tokens = s->num_tokens;
  a.block_size = s->block_size;
  a.part_tokens = 0;
  a.max_parts = 1;
  if (sp.max_parts > 1) {
    a.part_tokens = sp.part_tokens;
    a.max_parts = sp.max_parts;
    a.part_ml = static_cast<float*>(workspace);
    a.part_o = static_cast<char*>(workspace) + sp.ml_bytes;
    a.part_half = sp.part_half ? 1 : 0;
  }
  return from_hip(pa::launch_multi_query(s->block_size, group, a,
                                         static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pa_status_t pa_multi_query(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* query_start, float scale, void* out,
                           const pa_multi_query_shape_t* s, void* stream) {
  pa_status_t st = check_mq_shape(s);
  if (st != PA_OK) return st;
  return multi_query_impl(q, k_pool, v_pool, block_tables, seq_lens, query_start, scale, out, s,
                          MqSplit{}, nullptr, stream);
}

size_t pa_multi_query_workspace_bytes(const pa_multi_query_shape_t* shape,
                                      int32_t partition_tokens) {
  MqSplit sp;
  if (mq_split_plan(shape, partition_tokens, &sp) != PA_OK) return 0;
  return sp.ml_bytes + sp.o_bytes;
}

pa_status_t pa_multi_query_split(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* seq_lens,
                                 const int32_t* query_start, float scale, void* out,
                                 const pa_multi_query_shape_t* shape, int32_t partition_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  MqSplit sp;
  pa_status_t st = mq_split_plan(shape, partition_tokens, &sp);
  if (st != PA_OK) return st;
  const size_t need = sp.ml_bytes + sp.o_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PA_EWORKSPACE;
  return multi_query_impl(q, k_pool, v_pool, block_tables, seq_lens, query_start, scale, out,
                          shape, sp, workspace, stream);
}

static pa_status_t cache_impl(const void* k, const void* v, const int64_t* slot_mapping,
                              void* k_pool, void* v_pool, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t dtype, const pa::AppendArgs& ap,
                              void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0 || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return PA_EINVAL;
  if ((head_dim * eb) % 16 != 0) return PA_EINVAL;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PA_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_EINVAL;
  pa::CacheArgs a{};
  a.k = k;
  a.v = v;
  a.slots = slot_mapping;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_slots = (int64_t)num_blocks * block_size;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.row_chunks = head_dim * eb / 16;
  a.block_size = block_size;
  a.append = ap;
  return from_hip(pa::launch_reshape_and_cache(a, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping,
                                 void* k_pool, void* v_pool, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t dtype, void* stream) {
  return cache_impl(k, v, slot_mapping, k_pool, v_pool, num_tokens, num_kv_heads, head_dim,
                    block_size, num_blocks, dtype, pa::AppendArgs{}, stream);
}

static pa_status_t append_args(int32_t* block_tables, int32_t* seq_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, pa::AppendArgs* ap) {
  if (num_seqs > 0 && (!block_tables || !seq_lens)) return PA_EINVAL;
  if (max_blocks_per_seq <= 0) return PA_EINVAL;
  ap->block_tables = block_tables;
  ap->seq_lens = seq_lens;
  ap->max_blocks = max_blocks_per_seq;
  return PA_OK;
}

pa_status_t pa_append_tokens(const void* k, const void* v, const int64_t* slot_mapping,
                             void* k_pool, void* v_pool, int32_t* block_tables,
                             int32_t* seq_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t dtype, void* stream) {
  pa::AppendArgs ap{};
  pa_status_t st = append_args(block_tables, seq_lens, num_seqs, max_blocks_per_seq, &ap);
  if (st != PA_OK) return st;
  return cache_impl(k, v, slot_mapping, k_pool, v_pool, num_seqs, num_kv_heads, head_dim,
                    block_size, num_blocks, dtype, ap, stream);
}

static pa_status_t copy_impl(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                             const int64_t* pairs, int32_t num_pairs, int64_t block_bytes,
                             int32_t src_blocks, int32_t dst_blocks, void* stream) {
  if (num_pairs < 0 || block_bytes <= 0 || block_bytes % 16 != 0 || src_blocks <= 0 ||
      dst_blocks <= 0)
    return PA_EINVAL;
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs || !aligned16(src_k) || !aligned16(src_v) ||
      !aligned16(dst_k) || !aligned16(dst_v))
    return PA_EINVAL;
  pa::CopyArgs a{};
  a.src_k = src_k;
  a.src_v = src_v;
  a.dst_k = dst_k;
  a.dst_v = dst_v;
  a.pairs = pairs;
  a.block_chunks = block_bytes / 16;
  a.num_pairs = num_pairs;
  a.src_blocks = src_blocks;
  a.dst_blocks = dst_blocks;
  return from_hip(pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

static pa_status_t cache_e4m3_impl(const void* k, const void* v, const int64_t* slot_mapping,
                                   void* k_pool, void* v_pool, int32_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, float k_scale, float v_scale,
                                   const pa::AppendArgs& ap, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 16 != 0 ||
      block_size <= 0 || num_blocks <= 0)
    return PA_EINVAL;
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.0f || v_scale <= 0.0f)
    return PA_EINVAL;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PA_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_EINVAL;
  pa::CacheArgs8 a{};
  a.k = k;
  a.v = v;
  a.slots = slot_mapping;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_slots = (int64_t)num_blocks * block_size;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.row_groups = head_dim / 8;
  a.block_size = block_size;
  a.append = ap;
  return from_hip(pa::launch_reshape_and_cache_e4m3(a, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_reshape_and_cache_e4m3(const void* k, const void* v, const int64_t* slot_mapping,
                                      void* k_pool, void* v_pool, int32_t num_tokens,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, float k_scale, float v_scale,
                                      void* stream) {
  return cache_e4m3_impl(k, v, slot_mapping, k_pool, v_pool, num_tokens, num_kv_heads, head_dim,
                         block_size, num_blocks, k_scale, v_scale, pa::AppendArgs{}, stream);
}

pa_status_t pa_append_tokens_e4m3(const void* k, const void* v, const int64_t* slot_mapping,
                                  void* k_pool, void* v_pool, int32_t* block_tables,
                                  int32_t* seq_lens, int32_t num_seqs,
                                  int32_t max_blocks_per_seq, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  float k_scale, float v_scale, void* stream) {
  pa::AppendArgs ap{};
  pa_status_t st = append_args(block_tables, seq_lens, num_seqs, max_blocks_per_seq, &ap);
  if (st != PA_OK) return st;
  return cache_e4m3_impl(k, v, slot_mapping, k_pool, v_pool, num_seqs, num_kv_heads, head_dim,
                         block_size, num_blocks, k_scale, v_scale, ap, stream);
}

pa_status_t pa_copy_blocks(void* k_pool, void* v_pool, const int64_t* pairs, int32_t num_pairs,
                           int64_t block_bytes, int32_t num_blocks, void* stream) {
  return copy_impl(k_pool, v_pool, k_pool, v_pool, pairs, num_pairs, block_bytes, num_blocks,
                   num_blocks, stream);
}

// A pool the swap kernel may touch: device memory, or pinned host memory
// mapped into the device's address space at the same address. Pageable host
// memory (unknown to HIP) is refused before any launch.
static bool device_reachable(const void* p) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error of the failed query
    return false;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) return true;
  if (attr.type == hipMemoryTypeHost) return attr.devicePointer == p;
  return false;
}

pa_status_t pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                           const int64_t* pairs, int32_t num_pairs, int64_t block_bytes,
                           int32_t src_num_blocks, int32_t dst_num_blocks, void* stream) {
  if (num_pairs > 0) {
    for (const void* p : {src_k, src_v, static_cast<const void*>(dst_k),
                          static_cast<const void*>(dst_v), static_cast<const void*>(pairs)})
      if (p && !device_reachable(p)) return PA_EINVAL;
  }
  return copy_impl(src_k, src_v, dst_k, dst_v, pairs, num_pairs, block_bytes, src_num_blocks,
                   dst_num_blocks, stream);
}

pa_status_t pa_device_errors(uint32_t* flags, void* stream) {
  if (!flags) return PA_EINVAL;
  *flags = 0;
  hipError_t e = pa::read_and_clear_errors(flags, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return from_hip(e);
  return *flags ? PA_EDEVICE : PA_OK;
}

const char* pa_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

const char* pa_status_str(pa_status_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_EINVAL: return "PA_EINVAL: invalid argument";
    case PA_EUNSUPPORTED: return "PA_EUNSUPPORTED: shape not built";
    case PA_EWORKSPACE: return "PA_EWORKSPACE: workspace missing or too small";
    case PA_ENOBLOCKS: return "PA_ENOBLOCKS: free pool exhausted";
    case PA_EREFCOUNT: return "PA_EREFCOUNT: block released more than referenced";
    case PA_EHIP: return "PA_EHIP: HIP runtime call failed";
    case PA_EDEVICE: return "PA_EDEVICE: out-of-range device index";
  }
  return "unknown pa_status_t";
}

}  // extern "C"
