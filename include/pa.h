/*
 * pa.h — C ABI of libpa: paged KV-cache decode attention for gfx950.
 *
 * Sources (page title, then the section that defines the operation):
 *   [Vij] "PagedAttention Explained: KV Blocks, Allocation, and Sharing"
 *   [FP]  "PagedAttention & vLLM"
 *   [ZQ]  "Walk through paged attention end to end, page table, block lookup,
 *         and how it enables higher throughput"
 *   [N4N] "What is PagedAttention and how does it manage KV cache"
 *
 * Conventions for every call below
 *   - Pointers marked [dev] are device memory on the current HIP device;
 *     [host] pointers are host memory. All buffers are owned by the caller;
 *     libpa never allocates, frees or retains device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     GPU calls only enqueue work on it and return; stream order makes a
 *     write (pa_reshape_and_cache, pa_copy_blocks) visible to a later
 *     pa_decode on the same stream.
 *   - Every call returns a pa_status_t. Host-visible arguments are checked
 *     before anything is enqueued; on any error nothing is enqueued.
 *   - Device-resident indices (block ids, slots, copy pairs, lengths) cannot
 *     be checked on the host without a sync. The kernels check each one
 *     against the sizes passed here, never access memory outside the
 *     buffers described, skip the offending work item and raise a bit in a
 *     per-device error word read by pa_device_errors().
 *   - Element types: PA_F32 (float) or PA_BF16 (bfloat16 bit patterns).
 *     q, the pools, new k/v and out share one type. Pointers must be
 *     16-byte aligned; head_dim * element size must be a multiple of 16.
 *
 * KV pool layout (one pool for K and one for V, per layer):
 *   pool[num_blocks][num_kv_heads][block_size][head_dim], row-major.
 *   A block holds block_size consecutive token positions of one sequence;
 *   inside a block the tokens of one head are contiguous ([FP] "The
 *   insight: KV cache as virtual memory"; [N4N] "How PagedAttention works").
 *   Slot s names position (block s / block_size, offset s % block_size).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype_t;

typedef enum {
  PA_OK = 0,
  PA_EINVAL = 1,        /* bad argument (null pointer, size, alignment)        */
  PA_EUNSUPPORTED = 2,  /* valid but not built (dtype/head_dim/block_size/G)   */
  PA_EWORKSPACE = 3,    /* workspace missing or smaller than required          */
  PA_ENOBLOCKS = 4,     /* block manager: free pool exhausted, state unchanged */
  PA_EREFCOUNT = 5,     /* block manager: release of an unreferenced block     */
  PA_EHIP = 6,          /* a HIP runtime call failed                           */
  PA_EDEVICE = 7        /* a kernel met an out-of-range device index           */
} pa_status_t;

/* Bits of the device error word (pa_device_errors). */
#define PA_DEVERR_BLOCK_ID 0x1u   /* block table entry outside [0, num_blocks) */
#define PA_DEVERR_SEQ_LEN 0x2u    /* seq_len < 0, > max_seq_len, or > table   */
#define PA_DEVERR_SLOT 0x4u       /* slot >= num_blocks * block_size, or an
                                     appended slot that does not fit its
                                     sequence's position (pa_append_tokens) */
#define PA_DEVERR_COPY_PAIR 0x8u  /* copy/swap pair id outside its pool         */
#define PA_DEVERR_QUERY 0x10u     /* multi-query: bad query range or length    */
#define PA_DEVERR_PREFIX 0x20u    /* shared-prefix decode: bad group or prefix  */
#define PA_DEVERR_PLAN 0x40u      /* work plan entry: bad sequence, length or partition */

/* Decode kernel variants (pa_decode_shape_t.variant). */
#define PA_VARIANT_AUTO 0   /* library's choice for the shape                     */
#define PA_VARIANT_VALU 1   /* q.K and P.V on the vector ALUs                     */
#define PA_VARIANT_MFMA 2   /* matrix cores; bf16, head_dim 128. Group 1, 2, 4:
                               q.K on matrix cores, P.V on the vector ALUs (the
                               default there). Group 8, 16 (block size 16-128):
                               the multi-token kernel with one token per
                               sequence, both products on matrix cores (the
                               default there, ~2.5x the vector kernel)        */
/* Hint OR-ed into pa_decode_shape_t.variant: sequences of the batch share
 * physical blocks (samples forked from one prompt, [FP] "Copy-on-write
 * sharing"). The group 1, 2, 4 matrix-core kernel then loads K/V with the
 * plain cache policy, so that a shared block read by one sequence is still
 * in L2 for the next; without it K/V loads stream (non-temporal), which is
 * faster when every block belongs to one sequence. Results are identical
 * either way. */
#define PA_DECODE_SHARED_KV 0x100
/* Option OR-ed into pa_decode_shape_t.variant (bf16 q/out, group 1, 2 or 4
 * on the matrix cores): partitions of 256 or more positions store their
 * normalised partial output in bf16 instead of fp32 (the (max, exp-sum)
 * statistics and the merge stay fp32). This halves the partial-output bytes
 * but adds a rounding of each partial: the output may then differ from the
 * exact result by up to 2^-8 * sum_j w_j |o_j| (w_j = partition j's weight in
 * the merge, o_j its partial output), which is far above the bf16 tolerance
 * when partials of opposite sign cancel. Off by default: partials are fp32
 * and the merge adds only fp32 rounding. */
#define PA_DECODE_HALF_PARTIALS 0x200

/* Shape of one pa_decode call. */
typedef struct {
  int32_t num_seqs;           /* B                                             */
  int32_t num_q_heads;        /* Hq                                            */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0, group G = Hq / Hkv         */
  int32_t head_dim;           /* D: 64 or 128                                  */
  int32_t block_size;         /* tokens per block: 8, 16, 32, 64 or 128 with
                                 PA_VARIANT_MFMA; 16 or 32 with PA_VARIANT_VALU */
  int32_t num_blocks;         /* physical blocks in each pool                  */
  int32_t max_blocks_per_seq; /* row stride (entries) of block_tables          */
  int32_t max_seq_len;        /* host bound on every seq_lens[i]; sizes the
                                 grid and the workspace                        */
  int32_t partition_tokens;   /* context partition length: 0 = automatic (512;
                                 1024 for 8-bit pools, when G is 8 or 16 on
                                 the matrix cores, and when max_seq_len is
                                 above 8192),
                                 -1 = one partition per sequence, else a
                                 positive multiple of block_size               */
  int32_t dtype;              /* pa_dtype_t                                    */
  int32_t variant;            /* PA_VARIANT_*, optionally | PA_DECODE_SHARED_KV
                                 | PA_DECODE_HALF_PARTIALS                     */
} pa_decode_shape_t;

/* Bytes of scratch workspace pa_decode needs for `shape`: the partial softmax
 * statistics and the normalised partial outputs (fp32-sized slots; bf16
 * data with PA_DECODE_HALF_PARTIALS), merged in fp32. 0 if the shape is
 * invalid. */
size_t pa_decode_workspace_bytes(const pa_decode_shape_t* shape);

/*
 * pa_decode — paged decode attention (one new query token per sequence).
 *
 * [ZQ] single-decode-step pseudo-code and "Red flags"; [Vij] "Borrow the
 * abstraction"; [N4N] "How PagedAttention works". For sequence i and query
 * head h (KV head g = h / G):
 *     for p < seq_lens[i]:  b = block_tables[i][p / bs], o = p % bs
 *                           s_p = scale * dot(q[i][h], k_pool[b][g][o])
 *     out[i][h] = sum_p softmax(s)_p * v_pool[b][g][o]
 * seq_lens counts every cached token including the one just written; a
 * length of 0 gives zeros. Positions >= seq_lens[i] and table entries past
 * ceil(seq_lens[i] / bs) are never read, so slack slots and -1 padding are
 * harmless. The context is processed in partitions of partition_tokens
 * positions whose softmax statistics are merged by the log-sum-exp identity
 * (pa_decode_partition then pa_decode_reduce).
 *
 *   q             [dev] [B][Hq][D]
 *   k_pool,v_pool [dev] [num_blocks][Hkv][bs][D]
 *   block_tables  [dev] int32 [B][max_blocks_per_seq], -1 = unallocated
 *   seq_lens      [dev] int32 [B]
 *   scale         softmax scale applied to q.k (e.g. 1/sqrt(D))
 *   out           [dev] [B][Hq][D], written; rounded to nearest-even for bf16
 *   work_plan     [dev] NULL (with num_units 0) for the full grid, or a work
 *                 plan from pa_decode_plan and its unit count (below)
 *   workspace     [dev] >= pa_decode_workspace_bytes(shape) bytes
 */
pa_status_t pa_decode(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens, float scale,
                      void* out, const pa_decode_shape_t* shape, const int32_t* work_plan,
                      int32_t num_units, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same operation, arguments and outputs as pa_decode (the
 * same kernels, bit-identical results) without the workspace arguments: the
 * partials live in a device array inside libpa, PA_NOALLOC_SCRATCH_BYTES per
 * GPU, which each GPU holds from the library's first call on it until the
 * process ends. The call allocates nothing.
 *   - PA_EWORKSPACE (nothing enqueued) if pa_decode_workspace_bytes(shape)
 *     exceeds PA_NOALLOC_SCRATCH_BYTES (256 sequences x 32 query heads x 8 KV
 *     heads x head_dim 128, for instance, fit 15 partitions: 7,680 positions
 *     at 512 per partition).
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     on one GPU (different streams, or threads without ordering) race and
 *     their outputs are undefined. Calls ordered on one stream are safe. No
 *     part of the array needs to start at zero: a call writes every partial
 *     it reads.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status_t pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens, float scale,
                              void* out, const pa_decode_shape_t* shape, void* stream);

/* First half of pa_decode: one workgroup per (sequence, KV head, partition)
 * writes that partition's max score, exp-sum and normalised partial output
 * to `workspace`; a sequence with a single partition gets its final `out`
 * row directly. Same arguments as pa_decode. */
pa_status_t pa_decode_partition(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                float scale, void* out, const pa_decode_shape_t* shape,
                                const int32_t* work_plan, int32_t num_units, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Work plans: the decode's grid built on the host from the lengths.
 *
 * Same operation as pa_decode (same definition and citations). Without a
 * plan the grid covers every (sequence, partition) pair up to max_seq_len,
 * and the pairs past a sequence's own length exit at once. When the caller
 * knows the lengths on the host (its block manager produced them),
 * pa_decode_plan lists only the pairs that hold positions: every full
 * partition first, in (sequence, partition) order, then each sequence's
 * last, shorter partition, longest first (an empty sequence gets one unit
 * that writes its zeros). A decode call given the plan (work_plan and
 * num_units of pa_decode, pa_decode_partition, the _e4m3 forms and
 * pa_decode_shared_prefix) launches one workgroup per (unit, KV head) in
 * that order. Each unit computes exactly what it computes without the plan,
 * so the outputs are bit-identical.
 *
 *   pa_decode_plan_capacity: units a plan for `shape` can hold at most
 *     (num_seqs x partitions of max_seq_len); 0 if the shape is invalid.
 *   pa_decode_plan: seq_lens [host] int32 [B], the same values the device
 *     copy will hold; walk_start [host] int32 [B] or NULL: the partitions of
 *     sequence i tile positions [walk_start[i], seq_lens[i]) (for
 *     pa_decode_shared_prefix: its prefix_lens; NULL = 0 for the other
 *     calls); work_plan [host] int32 [capacity][4] receives one entry
 *     (sequence, partition, that sequence's length, its walk start) per
 *     unit; *num_units [host] receives their count. A walk that starts at
 *     its sequence's end gets no unit. PA_EINVAL if a length is negative or
 *     above min(max_seq_len, max_blocks_per_seq * block_size), a start is
 *     negative or past its length, or capacity is too small. Shapes with 8
 *     or 16 query heads per KV head on the matrix cores (the multi-token
 *     per-tile kernel) take plans too: one wave per unit.
 *   In a decode call, work_plan [dev] is the pa_decode_plan output copied to
 *     the device (16-byte aligned) and num_units its count. The partition
 *     kernel takes each unit's length from its entry (seq_lens serves the
 *     merge and the unplanned path). An entry whose sequence is outside
 *     [0, B), whose length is negative or above the bound above, or whose
 *     partition holds no position is skipped and raises PA_DEVERR_PLAN. A
 *     plan built from other lengths (or starts) than the device's leaves
 *     outputs undefined (a partition missing from it is never computed, and
 *     nothing is read outside the buffers). pa_decode_reduce completes a
 *     planned pa_decode_partition call as it does an unplanned one.
 */
int64_t pa_decode_plan_capacity(const pa_decode_shape_t* shape);
pa_status_t pa_decode_plan(const pa_decode_shape_t* shape, const int32_t* seq_lens,
                           const int32_t* walk_start, int32_t* work_plan, int64_t capacity,
                           int32_t* num_units);

/*
 * pa_decode_shared_prefix — pa_decode for a batch whose sequences come in
 * groups that share a prompt (samples forked from one parent: [FP]
 * "Copy-on-write sharing", [N4N] fork_block_table): sequences
 * group_start[k] .. group_start[k+1]-1 hold the same physical blocks in
 * their first prefix_lens[i] / block_size table entries. Same result as
 * pa_decode (to rounding), but each shared block is read once per group:
 * one pass per (group, KV head) attends the group's query rows (sequences x
 * heads of the group) to the prefix, one pass per (sequence, KV head) to
 * the positions after it, and a third kernel merges both passes' softmax
 * statistics and outputs (log-sum-exp, fp32).
 *
 *   shape          as pa_decode: bf16, head_dim 128, G in {1, 2, 4, 8, 16},
 *                  block size 16-128; both passes split their range into
 *                  partitions of partition_tokens positions (0: pa_decode's
 *                  automatic length); -1 is not accepted; of variant only
 *                  PA_DECODE_HALF_PARTIALS is read (it applies to the walks
 *                  after the prefix)
 *   group_start    [dev] int32 [num_groups + 1], non-decreasing, last <= B;
 *                  sequences outside every group need prefix_lens 0
 *   prefix_lens    [dev] int32 [B]: shared positions of each sequence, a
 *                  multiple of block_size, equal within a group, at most
 *                  seq_lens[i] and max_prefix_len; 0 = none
 *   max_group_size host bound on group sizes (sizes the grid)
 *   max_prefix_len host bound on prefix_lens, a multiple of block_size
 *   work_plan      [dev] NULL (num_units 0): the walks after the prefix run
 *                  over the full (sequence, partition) grid; else a work
 *                  plan from pa_decode_plan built with walk_start =
 *                  prefix_lens (host copies), for G in {1, 2, 4} only
 *   workspace      [dev] >= pa_decode_shared_prefix_workspace_bytes(shape,
 *                  max_group_size, max_prefix_len) bytes
 * A group whose members do not share the prefix (lengths differ, blocks
 * differ, or a member holds fewer positions), or a prefix length that is
 * not a multiple of block_size or exceeds max_prefix_len or its sequence,
 * is flagged (PA_DEVERR_PREFIX); the affected outputs are then undefined,
 * but every access stays inside the buffers.
 */
size_t pa_decode_shared_prefix_workspace_bytes(const pa_decode_shape_t* shape,
                                               int32_t max_group_size, int32_t max_prefix_len);
pa_status_t pa_decode_shared_prefix(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    float scale, void* out, const pa_decode_shape_t* shape,
                                    int32_t num_groups, const int32_t* group_start,
                                    const int32_t* prefix_lens, int32_t max_group_size,
                                    int32_t max_prefix_len, const int32_t* work_plan,
                                    int32_t num_units, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * 8-bit KV pools (FP8 E4M3). [ZQ] summary: paged attention composes with KV
 * quantization; the pages give no scheme, so this one is a reading: OCP FP8
 * E4M3 codes ("fn": no infinities, S.1111.111 = NaN, largest finite 448),
 * one positive float32 scale per pool; attention reads code value * scale.
 * Pools are [num_blocks][Hkv][bs][D] bytes; q and out stay bf16.
 *
 * pa_decode_e4m3 — pa_decode over 8-bit pools: s_p = scale * k_scale *
 * dot(q, code_K) and out = v_scale * sum_p softmax(s)_p code_V. shape->dtype
 * must be PA_BF16 (q, out), head_dim 128, group 1, 2 or 4, block size 16,
 * 32, 64 or 128; the matrix-core kernel runs whatever shape->variant says
 * (PA_VARIANT_VALU gives PA_EUNSUPPORTED; PA_DECODE_SHARED_KV applies as in
 * pa_decode). Workspace and work plan as pa_decode; the second half is
 * pa_decode_reduce unchanged. The automatic partition length of 8-bit pools
 * (1024) is not the one pa_decode_plan assumes for the shape, so with a work
 * plan shape->partition_tokens must be set explicitly, for the plan and for
 * the call; 0 then gives PA_EINVAL.
 */
pa_status_t pa_decode_e4m3(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens, float scale,
                           float k_scale, float v_scale, void* out,
                           const pa_decode_shape_t* shape, const int32_t* work_plan,
                           int32_t num_units, void* workspace, size_t workspace_bytes,
                           void* stream);
pa_status_t pa_decode_partition_e4m3(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_tables, const int32_t* seq_lens,
                                     float scale, float k_scale, float v_scale, void* out,
                                     const pa_decode_shape_t* shape, const int32_t* work_plan,
                                     int32_t num_units, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Second half of pa_decode: for every sequence with more than one partition,
 * out[i][h] = sum_j w_j o_j / sum_j w_j with w_j = l_j * exp(m_j - max_j m_j),
 * read from the workspace pa_decode_partition filled. */
pa_status_t pa_decode_reduce(const int32_t* seq_lens, void* out,
                             const pa_decode_shape_t* shape, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Shape of one pa_multi_query call. */
typedef struct {
  int32_t num_seqs;           /* B                                             */
  int32_t num_q_heads;        /* Hq                                            */
  int32_t num_kv_heads;       /* Hkv; G = Hq / Hkv in {1, 2, 4, 8, 16}          */
  int32_t head_dim;           /* D: 128                                        */
  int32_t block_size;         /* 16, 32, 64 or 128                             */
  int32_t num_blocks;         /* physical blocks in each pool                  */
  int32_t max_blocks_per_seq; /* row stride (entries) of block_tables          */
  int32_t max_seq_len;        /* host bound on every seq_lens[i]               */
  int32_t max_query_len;      /* host bound on query tokens per sequence;
                                 sizes the grid                                */
  int32_t num_tokens;         /* T = query_start[B], rows of q and out         */
  int32_t dtype;              /* PA_BF16                                       */
} pa_multi_query_shape_t;

/*
 * pa_multi_query — attention of several new query tokens per sequence (a
 * prefill chunk, or speculative tokens to verify) over the paged cache.
 *
 * [ZQ] comparison table: the paged kernel is FlashAttention with a
 * block-table dereference (pseudo-code: "Real kernels fuse this with
 * FlashAttention tiling"). Sequence i's query tokens are rows
 * query_start[i] .. query_start[i+1]-1 of q; they are its last Tq_i
 * positions and are already in the cache (pa_reshape_and_cache first), so
 * seq_lens[i] counts them. Token t sits at position p = seq_lens[i] - Tq_i
 * + t and, for every query head h (KV head h / G), attends causally to
 * positions 0 .. p:
 *     out[row][h] = sum_{p' <= p} softmax_p'(scale * q[row][h] . K[p']) V[p']
 * With one token per sequence this is pa_decode. Both products run on the
 * matrix cores with fp32 accumulation. From 128 query rows per KV head
 * (max_query_len * G >= 128) the call makes two launches on `stream`: the
 * first holds P and V in fp16 and serves the tiles whose context holds V
 * values within +-8 only; a tile with a larger (or non-finite) V value
 * writes nothing there, and the second launch, which otherwise exits at
 * once, redoes the call with P as two bf16 terms (as the call takes for
 * fewer rows). A sequence whose query range is invalid (Tq_i < 0,
 * Tq_i > seq_lens[i], > max_query_len, or past num_tokens) is skipped and
 * flagged (PA_DEVERR_QUERY).
 *
 *   q, out        [dev] [num_tokens][Hq][D] bf16
 *   k_pool,v_pool [dev] [num_blocks][Hkv][bs][D] bf16
 *   block_tables  [dev] int32 [B][max_blocks_per_seq]
 *   seq_lens      [dev] int32 [B]
 *   query_start   [dev] int32 [B + 1], non-decreasing, query_start[0] = 0
 */
pa_status_t pa_multi_query(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* query_start, float scale, void* out,
                           const pa_multi_query_shape_t* shape, void* stream);

/* Bytes of workspace pa_multi_query_split needs for `shape` with context
 * partitions of `partition_tokens` positions (0 = 1024): per query row
 * (token, query head) and partition, the (max, exp-sum) pair in fp32 and
 * the normalised partial output in bf16. 0 if nothing would be split or the
 * arguments are invalid (partition_tokens must be a positive multiple of
 * 16). */
size_t pa_multi_query_workspace_bytes(const pa_multi_query_shape_t* shape,
                                      int32_t partition_tokens);

/*
 * pa_multi_query_split — pa_multi_query with the context split into
 * partitions of `partition_tokens` positions for chunks of few query rows
 * (under 128 per KV head: speculative tokens), so that a sequence's context
 * is walked by many workgroups at once; a second kernel merges the
 * partitions' softmax statistics and outputs exactly (log-sum-exp) in fp32.
 * Larger chunks already have enough rows in flight and run unsplit, as in
 * pa_multi_query. Same result (to rounding) and arguments as
 * pa_multi_query, plus:
 *   partition_tokens  positions per partition, a positive multiple of 16,
 *                     or 0 for 1024
 *   workspace         [dev] >= pa_multi_query_workspace_bytes(shape,
 *                     partition_tokens) bytes, 16-byte aligned (PA_EWORKSPACE
 *                     otherwise); caller-owned, overwritten
 */
pa_status_t pa_multi_query_split(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* seq_lens,
                                 const int32_t* query_start, float scale, void* out,
                                 const pa_multi_query_shape_t* shape, int32_t partition_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_reshape_and_cache — write new tokens' K and V rows into their slots.
 *
 * [ZQ] pseudo-code (the new token's K/V go to block table[-1] at offset
 * pos % bs) and comparison table (generation writes into the current
 * block). For t < num_tokens with slot_mapping[t] >= 0:
 *     k_pool[slot / bs][h][slot % bs][:] = k[t][h][:]   for every h < Hkv
 * and the same for v. Bitwise copy. slot < 0 means "no write" (padding).
 * Slots must be distinct; two tokens writing one slot race.
 *
 *   k, v          [dev] [num_tokens][Hkv][D]
 *   slot_mapping  [dev] int64 [num_tokens]
 *   k_pool,v_pool [dev] [num_blocks][Hkv][bs][D]
 */
pa_status_t pa_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping,
                                 void* k_pool, void* v_pool, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, int32_t dtype, void* stream);

/*
 * pa_reshape_and_cache_e4m3 — the slot write into 8-bit pools. For t with
 * slot_mapping[t] >= 0 and every head h and dim d:
 *     k_pool[slot / bs][h][slot % bs][d] = E4M3(k[t][h][d] / k_scale)
 * (and v with v_scale), where E4M3 picks the code nearest to the exact
 * quotient (ties to the even mantissa), saturating at +-448, NaN to 0x7F
 * with the input's sign. k, v [dev] bf16 [num_tokens][Hkv][D];
 * head_dim a multiple of 16; scales finite and positive.
 */
pa_status_t pa_reshape_and_cache_e4m3(const void* k, const void* v, const int64_t* slot_mapping,
                                      void* k_pool, void* v_pool, int32_t num_tokens,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, float k_scale, float v_scale,
                                      void* stream);

/*
 * pa_append_tokens — one decode step's append for every sequence, on the
 * device: the slot write of pa_reshape_and_cache plus the device copies of
 * the block table and the length kept in step with the host block manager.
 *
 * [ZQ] single-decode-step pseudo-code: take a block when the position starts
 * one, put the new K/V at (last block, position % bs), and the sequence
 * grows by one token. The host decides (pa_bm_append_slots gives each
 * sequence its slot, after any new block or copy-on-write); this call
 * applies the decision to device-resident tables and lengths, so a decode
 * loop need not upload whole tables every step. Token t belongs to sequence
 * t. For t < num_seqs with slot_mapping[t] >= 0 and p = seq_lens[t]:
 *     pools[slot / bs][h][slot % bs][:] = k[t][h][:], v[t][h][:]   (all h)
 *     block_tables[t][p / bs] = slot / bs;   seq_lens[t] = p + 1
 * That table entry is the new block when p % bs == 0, the replacement block
 * after a copy-on-write, and otherwise the entry already there. Table
 * changes of fork, free and swap are not appends: upload those rows.
 * slot < 0: nothing happens for that sequence. A position p < 0 or past the
 * table (p / bs >= max_blocks_per_seq), or a slot with slot % bs != p % bs,
 * raises PA_DEVERR_SLOT and leaves table and length unchanged (the K/V row
 * is still written to its slot).
 *
 *   k, v          [dev] [num_seqs][Hkv][D]
 *   slot_mapping  [dev] int64 [num_seqs]
 *   block_tables  [dev] int32 [num_seqs][max_blocks_per_seq], updated
 *   seq_lens      [dev] int32 [num_seqs], updated
 *   pools, sizes, dtype and stream as pa_reshape_and_cache; the _e4m3 form
 *   writes 8-bit pools as pa_reshape_and_cache_e4m3 does.
 */
pa_status_t pa_append_tokens(const void* k, const void* v, const int64_t* slot_mapping,
                             void* k_pool, void* v_pool, int32_t* block_tables,
                             int32_t* seq_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t dtype, void* stream);
pa_status_t pa_append_tokens_e4m3(const void* k, const void* v, const int64_t* slot_mapping,
                                  void* k_pool, void* v_pool, int32_t* block_tables,
                                  int32_t* seq_lens, int32_t num_seqs,
                                  int32_t max_blocks_per_seq, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  float k_scale, float v_scale, void* stream);

/*
 * pa_copy_blocks — copy-on-write duplication of whole physical blocks.
 *
 * [FP] "Copy-on-write sharing": a sequence about to write into a block it
 * shares gets a private copy of that one block first. For each pair n:
 *     k_pool[dst] = k_pool[src],  v_pool[dst] = v_pool[src]   (bitwise)
 * where (src, dst) = (pairs[2n], pairs[2n+1]). Destinations must be distinct
 * and must not appear as sources in the same call (pairs run concurrently).
 *
 *   k_pool,v_pool [dev] num_blocks blocks of block_bytes bytes each
 *   pairs         [dev] int64 [num_pairs][2]
 *   block_bytes   Hkv * bs * D * element size; a multiple of 16
 */
pa_status_t pa_copy_blocks(void* k_pool, void* v_pool, const int64_t* pairs, int32_t num_pairs,
                           int64_t block_bytes, int32_t num_blocks, void* stream);

/*
 * pa_swap_blocks — move whole blocks between two pool pairs: a device pool
 * and a swap pool in pinned host memory, either way.
 *
 * [N4N] "Why it matters for KV cache" (swapping and preemption: blocks are
 * evicted to CPU memory when GPU memory runs short and fetched back when the
 * request resumes). For each pair n, with (src, dst) = (pairs[2n],
 * pairs[2n+1]):
 *     dst_k[dst] = src_k[src],  dst_v[dst] = src_v[src]   (bitwise)
 * One kernel moves every pair: host memory is read or written by the GPU
 * over the host link, so host pools must be pinned, device-mapped memory
 * (hipHostMalloc, or a pinned torch tensor). Destinations must be distinct.
 *
 *   src_k,src_v   [dev or pinned host] src_num_blocks blocks of block_bytes
 *   dst_k,dst_v   [dev or pinned host] dst_num_blocks blocks of block_bytes
 *   pairs         [dev] int64 [num_pairs][2]; ids out of range are skipped
 *                 and flagged (PA_DEVERR_COPY_PAIR)
 */
pa_status_t pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                           const int64_t* pairs, int32_t num_pairs, int64_t block_bytes,
                           int32_t src_num_blocks, int32_t dst_num_blocks, void* stream);

/* Returns the current device's error word in *flags (PA_DEVERR_* bits,
 * 0 = clean) as it stands once the work already enqueued on `stream` has
 * finished, and clears it: a one-thread kernel on `stream` fetches and
 * clears the word in one atomic exchange, then the call waits for the
 * value. A bit raised meanwhile by work on another stream is kept for the
 * next call. Returns PA_EDEVICE if any bit was set, PA_EHIP if a HIP call
 * failed. Concurrent calls from several host threads race on the fetched
 * copy. */
pa_status_t pa_device_errors(uint32_t* flags, void* stream);

/* Human-readable name of a status code (static storage). */
const char* pa_status_str(pa_status_t status);

/* Name of the HIP error behind the calling thread's most recent PA_EHIP
 * (hipGetErrorName; static storage), "hipSuccess" if the thread has had
 * none. Diagnostic only: a failed HIP call leaves the operation's outputs
 * undefined whatever its name. */
const char* pa_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Host block manager: free pool, block tables, reference counts, fork and
 * copy-on-write decisions. Host memory only, no GPU calls, not thread-safe.
 *
 * [FP] "The insight: KV cache as virtual memory" (blocks taken from one
 * shared pool on demand, per-request block table); [ZQ] pseudo-code (a new
 * block exactly when the position to write starts a block); [N4N]
 * "How PagedAttention works" (BlockTable.append_token), "Prefix sharing"
 * (fork_block_table) and the chat example (finished requests return their
 * blocks at once); [Vij] "Shared blocks need ownership rules" and [FP]
 * "Copy-on-write sharing" (reference counts, copy before writing into a
 * shared block).
 *
 * Readings: a fork shares every parent block including a partial last
 * block; freeing a swapped-out sequence returns its swap blocks; within one batch, writers are served in order, so the last writer
 * into a shared block keeps the original; freed blocks rejoin the back of
 * the free list in table order; the free list hands out blocks front first.
 * ------------------------------------------------------------------------ */
typedef struct pa_bm pa_bm_t;

/* Creates a manager for `num_blocks` blocks of `block_size` tokens.
 * free_order [host]: a permutation of 0..num_blocks-1 giving the order in
 * which blocks are handed out, or NULL for 0, 1, 2, ... */
pa_status_t pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         pa_bm_t** out);
void pa_bm_destroy(pa_bm_t* bm);

/* Registers sequence `seq_id` already holding `num_tokens` tokens and gives
 * it ceil(num_tokens / block_size) blocks. PA_ENOBLOCKS leaves state as is. */
pa_status_t pa_bm_add_seq(pa_bm_t* bm, int32_t seq_id, int32_t num_tokens);

/* Reserves the next token position of each of the n sequences (each listed
 * at most once), in order. slots [host] int64[n] receives block * bs +
 * offset. cow_pairs [host] int64[2n] receives the (src, dst) block copies
 * that must run (pa_copy_blocks) before the slots are written; *num_cow is
 * their count. All or nothing: PA_ENOBLOCKS if the pool cannot cover the
 * whole batch, with no state change. */
pa_status_t pa_bm_append_slots(pa_bm_t* bm, const int32_t* seq_ids, int32_t n, int64_t* slots,
                               int64_t* cow_pairs, int32_t* num_cow);

/* Child `child_id` shares every block of `parent_id` (count + 1 each). */
pa_status_t pa_bm_fork(pa_bm_t* bm, int32_t parent_id, int32_t child_id);

/* Drops a sequence; blocks whose count reaches 0 return to the free list. */
pa_status_t pa_bm_free_seq(pa_bm_t* bm, int32_t seq_id);

/* Writes the block tables [host] int32[n][max_blocks] (-1 padded) and token
 * counts [host] int32[n] of the listed sequences. PA_EINVAL if a table is
 * longer than max_blocks. Either output may be NULL. */
pa_status_t pa_bm_export(const pa_bm_t* bm, const int32_t* seq_ids, int32_t n,
                         int32_t max_blocks, int32_t* tables, int32_t* lens);

/* Swap space for preemption ([N4N] "Why it matters for KV cache", swapping
 * and preemption; [ZQ] summary, "easy preemption"): `num_cpu_blocks` host
 * blocks with their own free list (0, 1, 2, ... handed out front first).
 * PA_EINVAL while a sequence is swapped out. */
pa_status_t pa_bm_set_swap_space(pa_bm_t* bm, int32_t num_cpu_blocks);

/* Moves every block of `seq_id` to swap space, in table order: pairs [host]
 * int64[2 * max_pairs] receives (device block, swap block) for pa_swap_blocks
 * (device pools -> host pools); *num_pairs their count. A device block still
 * shared by other sequences stays with them (count - 1); the others return
 * to the back of the free list. A swapped-out sequence cannot be appended
 * to, forked or exported. PA_ENOBLOCKS (swap space short) leaves state
 * unchanged. */
pa_status_t pa_bm_swap_out(pa_bm_t* bm, int32_t seq_id, int64_t* pairs, int32_t max_pairs,
                           int32_t* num_pairs);

/* Brings a swapped-out sequence back: each swap block, in table order, gets
 * a fresh device block from the free list; pairs receives (swap block,
 * device block) for pa_swap_blocks (host pools -> device pools); swap blocks
 * rejoin the back of the swap free list. PA_ENOBLOCKS leaves state
 * unchanged. */
pa_status_t pa_bm_swap_in(pa_bm_t* bm, int32_t seq_id, int64_t* pairs, int32_t max_pairs,
                          int32_t* num_pairs);

/* Free swap-space blocks; 1 if `seq_id` is swapped out, 0 if resident, -1 if
 * unknown. */
int32_t pa_bm_num_free_swap(const pa_bm_t* bm);
int32_t pa_bm_is_swapped(const pa_bm_t* bm, int32_t seq_id);

int32_t pa_bm_num_free(const pa_bm_t* bm);
/* Reference count of `block`, or -1 if out of range. */
int32_t pa_bm_refcount(const pa_bm_t* bm, int32_t block);
/* Token count of `seq_id`, or -1 if unknown. */
int32_t pa_bm_num_tokens(const pa_bm_t* bm, int32_t seq_id);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
