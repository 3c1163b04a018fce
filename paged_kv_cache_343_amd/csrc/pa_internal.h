// Internal interface between the C ABI (pa_api.cpp) and the gfx950 kernels
// (pa_kernels.hip). Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Floats per (sequence, KV head, partition) record of partial softmax
// statistics: one 128-byte line, room for (max, exp-sum) of 16 query heads.
constexpr int kMlRecord = 32;

// Everything one decode launch needs, passed by value as the kernel argument.
struct DecodeArgs {
  const void* q;              // [B][Hq][D]
  const void* k_pool;         // [NB][Hkv][bs][D]
  const void* v_pool;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* seq_lens;      // [B]
  void* out;                    // [B][Hq][D]
  float* part_ml;               // [B][Hkv][max_parts][kMlRecord]: per query head of the
                                //   group, max score (log2 units) then exp-sum; rest 0
  void* part_o;                 // [B][Hq][max_parts][D] fp32 slots: normalised partial
                                //   output (bf16 in a slot's first half, see part_half)
  float qscale;                 // softmax scale * log2(e) (* k_scale for 8-bit pools)
  float out_scale;              // v_scale for 8-bit pools
  int32_t part_half;            // partial outputs stored as bf16
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_seq_len;
  int32_t len_cap;              // min(max_seq_len, max_blocks * bs)
  int32_t part_tokens;          // partition length in positions (multiple of bs)
  int32_t max_parts;            // ceil(max_seq_len / part_tokens): partitions in the grid
  // shared-prefix decode: the walk of sequence i starts at pos_start[i] (a
  // multiple of block_size, at most max_prefix), its partitions fill partial
  // slots slot0 .. and always leave partials; the reduce also merges the
  // prefix pass's slots 0 .. ceil(pos_start[i] / part_tokens) - 1 (fp32)
  const int32_t* pos_start;     // [B] or null
  int32_t prefix_part_tokens;   // partition length of the prefix pass
  int32_t slot0;
  int32_t slot_stride;          // partial slots per row (0: max_parts)
  int32_t max_prefix;
  int32_t block_size;
  // host-built work plan (pa_decode_plan): the grid covers num_units
  // (sequence, partition) pairs x Hkv instead of B x max_parts x Hkv
  const int32_t* plan;          // [num_units][4] (sequence, partition, length, 0) or null
  int32_t num_units;
};

// Device copies of the block tables and lengths kept in step with the host
// block manager's append (token t = sequence t): null tables = no upkeep.
struct AppendArgs {
  int32_t* block_tables;        // [num_tokens][max_blocks]
  int32_t* seq_lens;            // [num_tokens]
  int32_t max_blocks;
};

struct CacheArgs {
  const void* k;                // [T][Hkv][D]
  const void* v;
  const int64_t* slots;         // [T]
  void* k_pool;
  void* v_pool;
  int64_t num_slots;            // num_blocks * block_size
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t row_chunks;           // 16-byte chunks per (token, head) row = D * elem / 16
  int32_t block_size;
  AppendArgs append;            // table / length upkeep (pa_append_tokens) or none
};

// Slot write into FP8 E4M3 pools from bf16 rows.
struct CacheArgs8 {
  const void* k;                // [T][Hkv][D] bf16
  const void* v;
  const int64_t* slots;         // [T]
  void* k_pool;                 // [NB][Hkv][bs][D] codes
  void* v_pool;
  int64_t num_slots;            // num_blocks * block_size
  float k_scale;                // a value x is stored as the code of x / k_scale
  float v_scale;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t row_groups;           // 8-element groups per row = D / 8
  int32_t block_size;
  AppendArgs append;
};

// Whole-block copies from (src_k, src_v) to (dst_k, dst_v): the same pools
// for copy-on-write, a device pool and a pinned host pool for swapping.
struct CopyArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int64_t* pairs;         // [N][2] (src block, dst block)
  int64_t block_chunks;         // 16-byte chunks per block
  int32_t num_pairs;
  int32_t src_blocks;           // blocks in the source pools
  int32_t dst_blocks;           // blocks in the destination pools
};

// Multi-token query launch (prefill chunk / speculative tokens).
struct MqArgs {
  const void* q;                // [T][Hq][D]
  const void* k_pool;           // [NB][Hkv][bs][D]
  const void* v_pool;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* seq_lens;      // [B], query tokens included
  const int32_t* query_start;   // [B + 1]
  void* out;                    // [T][Hq][D]
  float qscale;                 // softmax scale * log2(e)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t len_cap;              // min(max_seq_len, max_blocks * bs)
  int32_t max_query_len;
  int32_t num_tokens;           // T
  int32_t part_tokens;          // context partition length (0: one partition)
  int32_t max_parts;            // partitions of the longest context (1 if unsplit)
  float* part_ml;               // [T][Hq][max_parts][2]: max score (log2 units), exp-sum
  void* part_o;                 // [T][Hq][max_parts][D]: normalised partial output, bf16
                                //   if part_half, else fp32
  int32_t part_half;
  int32_t decode_mode;          // one query token per sequence: token i of sequence i,
                                //   query_start unused, pa_decode's length rules
  // shared-prefix decode (mode 2: one pass per group over the shared prefix,
  // mode 3: one pass per sequence over the rest); 0 otherwise
  int32_t mode;
  const int32_t* group_start;   // [num_groups + 1] (mode 2)
  const int32_t* prefix_lens;   // [B] shared positions of each sequence (modes 2, 3)
  int32_t suffix_slot0;         // first partial slot of the per-sequence pass
  int32_t prefix_part_tokens;   // partition length of the prefix pass (mode 2)
  int32_t max_prefix;           // host bound on prefix_lens (sizes the prefix slots)
  int32_t block_size;
  int32_t slot_stride;          // partial slots per row (0: max_parts)
  int32_t ml_records;           // mode 2: (max, exp-sum) in pa_decode's 128-byte records
  // decode mode over a host work plan (pa_decode_plan): [num_units][4]
  // (sequence, partition, length, 0), one wave each; null otherwise
  const int32_t* plan;
  int32_t num_units;
  // workgroup-tiled multi-token kernel: this call's ticket (set by its launcher)
  uint64_t fa_ticket;
};

// When the caller asks for bf16 partials (part_half), the decode kernels
// keep the partial output of a partition in bf16 if it covers at least this
// many positions and the output is bf16; shorter partials, those of the
// multi-token kernels, and all partials by default stay fp32.
constexpr int kHalfPartialMinTokens = 256;

// Kernel selection key for pa_decode_partition.
struct DecodeKey {
  int dtype;       // 0 f32, 1 bf16
  int head_dim;    // 64, 128
  int block_size;  // 16, 32
  int group;       // 1, 2, 4, 8
  int variant;     // 1 VALU, 2 MFMA
  bool kv_fp8;     // pools hold FP8 E4M3 codes (q, out bf16)
  bool cached_kv;  // blocks shared between sequences: plain (not streaming)
                   //   K/V loads in the matrix-core kernel
};

// Returns hipErrorInvalidValue (and launches nothing) if `key` has no kernel.
hipError_t launch_decode_partition(const DecodeKey& key, const DecodeArgs& args,
                                   hipStream_t stream);
bool decode_partition_supported(const DecodeKey& key);
hipError_t launch_decode_reduce(int dtype, int head_dim, const DecodeArgs& args,
                                hipStream_t stream);
hipError_t launch_reshape_and_cache(const CacheArgs& args, hipStream_t stream);
hipError_t launch_reshape_and_cache_e4m3(const CacheArgs8& args, hipStream_t stream);
bool multi_query_supported(int dtype, int head_dim, int block_size, int group);
hipError_t launch_multi_query(int block_size, int group, const MqArgs& args, hipStream_t stream);
// The two halves of the per-tile path: 16-row tiles (and context partitions
// when args.max_parts > 1), then the merge of the partitions.
hipError_t launch_multi_query_tiles(int block_size, int group, const MqArgs& args,
                                   hipStream_t stream);
hipError_t launch_multi_query_reduce(int group, const MqArgs& args, hipStream_t stream);
// Shared-prefix decode's two passes in one launch: the prefix pass (pre,
// mode 2, the per-tile kernel) and the per-sequence walks (walk, with
// pos_start; group 1, 2 or 4); the decode reduce merges them afterwards.
hipError_t launch_shared_prefix_decode(int block_size, int group, const MqArgs& pre,
                                       const DecodeArgs& walk, hipStream_t stream);
// True if chunks of up to max_query_len tokens run on the workgroup-tiled
// kernel (which never splits the context).
bool multi_query_tiled(int group, int max_query_len);
hipError_t launch_copy_blocks(const CopyArgs& args, hipStream_t stream);
// Fetches and clears the device error word in one atomic exchange, ordered
// after the work already enqueued on `stream`, and waits for the value.
hipError_t read_and_clear_errors(uint32_t* flags, hipStream_t stream);

// Workgroup size (waves) of the partition kernels.
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
constexpr int kDecodeWaves = PA_DECODE_WAVES;
// Waves per workgroup of the matrix-core decode kernel with 1, 2 or 4 query
// heads per KV head on large grids (small grids and its shared-prefix walk
// keep kDecodeWaves): two waves make twice the workgroups, each walking 16
// of a 512-position partition's 32 chunks, which evens out the end of the
// grid.
#ifndef PA_MFMA_DECODE_WAVES
#define PA_MFMA_DECODE_WAVES 2
#endif
constexpr int kMfmaDecodeWaves = PA_MFMA_DECODE_WAVES;
// Waves per workgroup of the partition merge (one wave per query head).
constexpr int kReduceWaves = 4;

}  // namespace pa
