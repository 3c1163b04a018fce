// Host block manager: free pool, per-sequence block tables, reference
// counts, fork and copy-on-write decisions. Host memory only.
//
// The pool hands out fixed-size blocks on demand ("PagedAttention & vLLM",
// "The insight: KV cache as virtual memory"); a sequence takes a new block
// exactly when the position it writes starts a block (the single decode
// step pseudo-code on the zenaique.com page); forks share blocks and a
// write into a block with more than one owner duplicates it first
// ("PagedAttention & vLLM", "Copy-on-write sharing"; n4n.ai "Prefix
// sharing"); finished sequences give their blocks straight back (n4n.ai,
// chat workload example).
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;               // front = next block handed out
  std::vector<int32_t> ref;                    // owners per physical block
  struct Seq {
    std::vector<int32_t> table;                // logical block -> physical id
    int32_t ntok = 0;
    uint64_t stamp = 0;                        // call that last listed it
    bool swapped = false;                      // table names swap-space blocks
  };
  int32_t num_cpu_blocks = 0;                  // swap space (host) blocks
  std::deque<int32_t> cpu_free;
  std::unordered_map<int32_t, Seq> seqs;
  uint64_t epoch = 0;                          // append call counter
  std::vector<Seq*> batch;                     // scratch of pa_bm_append_slots
  std::vector<int32_t> dropped;                // per block: references the batch
                                               //   being counted gives up
  std::vector<int32_t> touched;                // blocks with dropped != 0

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }
  // Blocks that appending one token to each of batch[0 .. n) takes: one per
  // position that starts a block, and one per write into a block that some
  // other holder still shares at that point. Writers into one shared block
  // are served in batch order and each copy gives up the writer's reference,
  // so the last holder writes in place and takes none.
  int64_t blocks_for_appends(int32_t n) {
    int64_t need = 0;
    if (dropped.size() != ref.size()) dropped.assign(ref.size(), 0);
    touched.clear();
    for (int32_t k = 0; k < n; ++k) {
      const Seq& s = *batch[(size_t)k];
      if (s.ntok % block_size == 0) {
        ++need;
        continue;
      }
      const int32_t b = s.table[s.ntok / block_size];
      if (ref[b] - dropped[b] > 1) {
        ++need;
        if (dropped[b]++ == 0) touched.push_back(b);
      }
    }
    for (int32_t b : touched) dropped[b] = 0;
    return need;
  }
};

static int64_t blocks_for(int64_t ntok, int32_t bs) { return (ntok + bs - 1) / bs; }

extern "C" {

pa_status_t pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         pa_bm_t** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PA_EINVAL;
  *out = nullptr;
  pa_bm* bm = new (std::nothrow) pa_bm;
  if (!bm) return PA_EINVAL;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t k = 0; k < num_blocks; ++k) {
      const int32_t b = free_order[k];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PA_EINVAL;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_bm_t* bm) { delete bm; }

pa_status_t pa_bm_add_seq(pa_bm_t* bm, int32_t seq_id, int32_t num_tokens) {
  if (!bm || num_tokens < 0) return PA_EINVAL;
  if (bm->seqs.count(seq_id)) return PA_EINVAL;
  const int64_t need = blocks_for(num_tokens, bm->block_size);
  if (need > (int64_t)bm->free_list.size()) return PA_ENOBLOCKS;
  pa_bm::Seq s;
  s.table.reserve((size_t)need);
  for (int64_t k = 0; k < need; ++k) s.table.push_back(bm->take());
  s.ntok = num_tokens;
  bm->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status_t pa_bm_append_slots(pa_bm_t* bm, const int32_t* seq_ids, int32_t n, int64_t* slots,
                               int64_t* cow_pairs, int32_t* num_cow) {
  if (!bm || n < 0 || (n > 0 && (!seq_ids || !slots || !cow_pairs)) || !num_cow)
    return PA_EINVAL;
  *num_cow = 0;
  // Validate the whole batch and count the blocks it needs before changing
  // anything, so that a failure leaves the state untouched. A sequence
  // listed twice is caught by its stamp (set to this call's epoch).
  std::vector<pa_bm::Seq*>& batch = bm->batch;
  batch.resize((size_t)n);
  const uint64_t epoch = ++bm->epoch;
  int64_t need = 0;
  for (int32_t k = 0; k < n; ++k) {
    auto it = bm->seqs.find(seq_ids[k]);
    if (it == bm->seqs.end() || it->second.stamp == epoch) return PA_EINVAL;
    if (it->second.ntok == INT32_MAX || it->second.swapped) return PA_EINVAL;
    it->second.stamp = epoch;
    batch[k] = &it->second;
  }
  need = bm->blocks_for_appends(n);
  if (need > (int64_t)bm->free_list.size()) return PA_ENOBLOCKS;
  const int32_t bs = bm->block_size;
  int32_t ncow = 0;
  for (int32_t k = 0; k < n; ++k) {
    pa_bm::Seq& s = *batch[k];
    const int32_t p = s.ntok;
    const int32_t lblk = p / bs, off = p % bs;
    if (off == 0) {
      s.table.push_back(bm->take());            // position starts a new block
    } else if (bm->ref[s.table[lblk]] > 1) {
      const int32_t src = s.table[lblk];        // shared: copy, then write
      const int32_t dst = bm->take();
      bm->ref[src] -= 1;
      s.table[lblk] = dst;
      cow_pairs[2 * ncow] = src;
      cow_pairs[2 * ncow + 1] = dst;
      ++ncow;
    }
    s.ntok = p + 1;
    slots[k] = (int64_t)s.table[lblk] * bs + off;
  }
  *num_cow = ncow;
  return PA_OK;
}

pa_status_t pa_bm_fork(pa_bm_t* bm, int32_t parent_id, int32_t child_id) {
  if (!bm) return PA_EINVAL;
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end() || bm->seqs.count(child_id) || it->second.swapped) return PA_EINVAL;
  pa_bm::Seq child = it->second;
  for (int32_t b : child.table) bm->ref[b] += 1;
  bm->seqs.emplace(child_id, std::move(child));
  return PA_OK;
}

pa_status_t pa_bm_free_seq(pa_bm_t* bm, int32_t seq_id) {
  if (!bm) return PA_EINVAL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_EINVAL;
  if (it->second.swapped) {
    for (int32_t c : it->second.table) bm->cpu_free.push_back(c);
    bm->seqs.erase(it);
    return PA_OK;
  }
  for (int32_t b : it->second.table)
    if (bm->ref[b] <= 0) return PA_EREFCOUNT;
  for (int32_t b : it->second.table) {
    if (--bm->ref[b] == 0) bm->free_list.push_back(b);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status_t pa_bm_export(const pa_bm_t* bm, const int32_t* seq_ids, int32_t n,
                         int32_t max_blocks, int32_t* tables, int32_t* lens) {
  if (!bm || n < 0 || max_blocks < 0 || (n > 0 && !seq_ids)) return PA_EINVAL;
  for (int32_t k = 0; k < n; ++k) {
    auto it = bm->seqs.find(seq_ids[k]);
    if (it == bm->seqs.end() || it->second.swapped) return PA_EINVAL;
    if ((int64_t)it->second.table.size() > max_blocks) return PA_EINVAL;
  }
  for (int32_t k = 0; k < n; ++k) {
    const pa_bm::Seq& s = bm->seqs.find(seq_ids[k])->second;
    if (tables) {
      int32_t* row = tables + (int64_t)k * max_blocks;
      const size_t len = s.table.size();
      if (len) std::memcpy(row, s.table.data(), len * sizeof(int32_t));
      std::fill(row + len, row + max_blocks, -1);
    }
    if (lens) lens[k] = s.ntok;
  }
  return PA_OK;
}

// Swapping ([N4N] "Why it matters for KV cache": blocks evicted to CPU memory
// under pressure and fetched back when the request resumes; [ZQ] summary:
// easy preemption). Swap space is a second pool of host blocks with its own
// free list, handed out front first; a swapped-out sequence's table names
// swap-space blocks until it is swapped back in.
pa_status_t pa_bm_set_swap_space(pa_bm_t* bm, int32_t num_cpu_blocks) {
  if (!bm || num_cpu_blocks < 0) return PA_EINVAL;
  for (const auto& kv : bm->seqs)
    if (kv.second.swapped) return PA_EINVAL;    // swap space in use
  bm->num_cpu_blocks = num_cpu_blocks;
  bm->cpu_free.clear();
  for (int32_t c = 0; c < num_cpu_blocks; ++c) bm->cpu_free.push_back(c);
  return PA_OK;
}

pa_status_t pa_bm_swap_out(pa_bm_t* bm, int32_t seq_id, int64_t* pairs, int32_t max_pairs,
                           int32_t* num_pairs) {
  if (!bm || !num_pairs) return PA_EINVAL;
  *num_pairs = 0;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || it->second.swapped) return PA_EINVAL;
  pa_bm::Seq& s = it->second;
  const int32_t n = (int32_t)s.table.size();
  if (n > max_pairs || (n > 0 && !pairs)) return PA_EINVAL;
  if (n > (int32_t)bm->cpu_free.size()) return PA_ENOBLOCKS;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t b = s.table[k];
    const int32_t c = bm->cpu_free.front();
    bm->cpu_free.pop_front();
    pairs[2 * k] = b;
    pairs[2 * k + 1] = c;
    // a block still shared by other sequences stays on the device for them
    if (--bm->ref[b] == 0) bm->free_list.push_back(b);
    s.table[k] = c;
  }
  s.swapped = true;
  *num_pairs = n;
  return PA_OK;
}

pa_status_t pa_bm_swap_in(pa_bm_t* bm, int32_t seq_id, int64_t* pairs, int32_t max_pairs,
                          int32_t* num_pairs) {
  if (!bm || !num_pairs) return PA_EINVAL;
  *num_pairs = 0;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || !it->second.swapped) return PA_EINVAL;
  pa_bm::Seq& s = it->second;
  const int32_t n = (int32_t)s.table.size();
  if (n > max_pairs || (n > 0 && !pairs)) return PA_EINVAL;
  if (n > (int32_t)bm->free_list.size()) return PA_ENOBLOCKS;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t c = s.table[k];
    const int32_t d = bm->take();
    pairs[2 * k] = c;
    pairs[2 * k + 1] = d;
    bm->cpu_free.push_back(c);
    s.table[k] = d;
  }
  s.swapped = false;
  *num_pairs = n;
  return PA_OK;
}

int32_t pa_bm_num_free_swap(const pa_bm_t* bm) { return bm ? (int32_t)bm->cpu_free.size() : -1; }

int32_t pa_bm_is_swapped(const pa_bm_t* bm, int32_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

int32_t pa_bm_num_free(const pa_bm_t* bm) { return bm ? (int32_t)bm->free_list.size() : -1; }

int32_t pa_bm_refcount(const pa_bm_t* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int32_t pa_bm_num_tokens(const pa_bm_t* bm, int32_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : it->second.ntok;
}

}  // extern "C"
