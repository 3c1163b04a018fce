"""CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link
or execute this module: only the tests, the smoke check of the entry script
and the bench's CPU-baseline leg use it. It shares no code with the HIP path
and never imports it.

What it computes, each piece written out plainly in float64 (inputs are
converted exactly from their fp32 or bf16 bits):

* allocation arithmetic: blocks a sequence needs, last-block slack, and the
  slot (physical block, offset) of a logical position;
* a block manager mirror: a free pool handing out blocks in a given order,
  per-sequence block tables grown one token at a time, reference counts,
  fork, copy-on-write on a write into a shared block, and freeing;
* decode attention: for every attended position p the block table is
  dereferenced at p // block_size and the row read at offset p % block_size,
  then exact softmax attention over those rows;
* the same attention split into fixed-length context partitions and combined
  by the log-sum-exp identity;
* attention of several new query tokens per sequence (a prefill chunk or
  speculative tokens) over the same paged cache, each token attending to
  every position up to and including its own;
* the slot write of new K/V rows and the whole-block copy, bit for bit;
* swapping: a second (host) pool with its own free list, a sequence's blocks
  moved out to it and back, and the block moves between the two pools;
* an 8-bit KV pool: the OCP FP8 E4M3 code of every value, the slot write that
  scales and rounds new rows into codes, and the dequantized pools that the
  ordinary decode then reads.

Sources (page title, then the section used):
  [Vij]  "PagedAttention Explained: KV Blocks, Allocation, and Sharing"
         (palashvij.pages.dev)
  [FP]   "PagedAttention & vLLM" (fp-ai-systems.pages.dev)
  [ZQ]   "Walk through paged attention end to end, page table, block
         lookup, and how it enables higher throughput" (zenaique.com)
  [N4N]  "What is PagedAttention and how does it manage KV cache"
         (n4n.ai blog)

Readings taken where the pages are silent (all listed with reasons in the
design notes of the repository):
  * the caller passes the softmax scale (the pages' pseudo-code applies none);
  * seq_lens counts every cached token including the one just written, so
    the new token attends to itself ([ZQ] pseudo-code writes first, then
    attends over seq_len + 1 positions);
  * GQA: query head h reads KV head h // (Hq / Hkv);
  * seq_len 0 gives an all-zero output;
  * a fork shares every block of the parent including a partial last block,
    and the first write into a block whose reference count exceeds one
    copies it first; writers are served in call order, so the last writer
    keeps the original block;
  * freed blocks return to the back of the free list, in table order;
  * a slot < 0 means "no write" (padding);
  * swap space hands out its blocks front first (0, 1, 2, ...); swapping a
    sequence out moves its table entries in order, a device block still
    shared by other sequences stays with them, the others and returned swap
    blocks rejoin the back of their free lists.

Every function here is pinned by tests against the pages' worked numbers,
closed forms, invariants, a library routine or brute force; none is
"parity unpinned".
"""
from __future__ import annotations

import math
from collections import deque

import numpy as np

__all__ = [
    "blocks_needed", "slack", "slot_of", "kv_bytes_per_token",
    "OracleNoBlocks", "OracleRefcountError", "OracleBlockManager",
    "as_f64", "positions_to_rows", "kv_head_of",
    "decode", "decode_one", "partition_partials", "combine_partials",
    "decode_partitioned", "reshape_and_cache", "copy_blocks", "swap_blocks",
    "multi_query", "E4M3_MAX", "e4m3_value", "e4m3_values", "e4m3_encode",
    "reshape_and_cache_e4m3", "dequantize_e4m3",
]


# --------------------------------------------------------------------------
# Allocation arithmetic
# --------------------------------------------------------------------------

def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks that hold `num_tokens` tokens: the count rounded up to whole
    blocks. [Vij] "Grow allocation with the sequence": 33 tokens in 16-token
    blocks take three blocks, 32 tokens take two."""
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens must be >= 0 and block_size > 0")
    return -(-int(num_tokens) // int(block_size))


def slack(num_tokens: int, block_size: int) -> int:
    """Unused token positions in the last block. [FP] "The insight: KV cache
    as virtual memory": the only waste left is in the last block, below one
    block's worth."""
    return blocks_needed(num_tokens, block_size) * block_size - int(num_tokens)


def slot_of(table, pos: int, block_size: int) -> int:
    """Flat slot of logical position `pos`: physical block table[pos // bs]
    at offset pos % bs, encoded as block * bs + offset. [ZQ] pseudo-code of
    the single decode step (the physical block and offset of a position)."""
    return int(table[pos // block_size]) * block_size + pos % block_size


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    """K and V bytes one token occupies across all layers: layers x 2 (K,V)
    x heads x head_dim x element bytes. [FP] "Worked example: naive vs
    paged" uses this for a 40-layer, 40-head, 128-dim model (~0.78 MB)."""
    return num_layers * 2 * num_kv_heads * head_dim * elem_bytes


# --------------------------------------------------------------------------
# Block manager mirror
# --------------------------------------------------------------------------

class OracleNoBlocks(RuntimeError):
    """The free pool cannot satisfy the request; nothing was changed."""


class OracleRefcountError(RuntimeError):
    """A block was released more often than it was referenced."""


class OracleBlockManager:
    """Free pool + per-sequence block tables + reference counts.

    [FP] "The insight": fixed-size blocks are taken from one shared pool on
    demand and mapped per request by a block table. [ZQ] pseudo-code: a new
    physical block is taken exactly when the position to write starts a
    block. [N4N] "How PagedAttention works" (BlockTable listing): the table
    maps logical block index to physical id and grows by one entry when the
    logical index reaches its length. [N4N] "Prefix sharing" and [FP]
    "Copy-on-write sharing": forks share physical blocks; a write into a
    shared block first duplicates that block. [N4N] chat example: freed
    blocks go straight back to the pool.
    """

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.free = deque(order)
        self.ref = [0] * self.num_blocks
        self.tables: dict[int, list[int]] = {}
        self.ntok: dict[int, int] = {}
        self.swap_free: deque = deque()
        self.swapped: set = set()

    # -- helpers ----------------------------------------------------------
    def _take(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, block: int) -> int:
        return self.ref[block]

    def table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def num_tokens(self, seq: int) -> int:
        return self.ntok[seq]

    # -- operations -------------------------------------------------------
    def add_seq(self, seq: int, num_tokens: int) -> None:
        """A new sequence holding `num_tokens` tokens gets exactly the blocks
        it needs, taken from the front of the free list."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        need = blocks_needed(num_tokens, self.block_size)
        if need > len(self.free):
            raise OracleNoBlocks(f"need {need}, free {len(self.free)}")
        self.tables[seq] = [self._take() for _ in range(need)]
        self.ntok[seq] = int(num_tokens)

    def _blocks_for_appends(self, seqs) -> int:
        """Blocks that appending one token to each listed sequence takes, in
        order: one for a position that starts a block, one for a write into
        a block still shared with another holder at that point (its copy
        gives up the writer's reference, so the last holder of a shared
        block writes in place and takes none)."""
        refs = dict()
        need = 0
        for s in seqs:
            p = self.ntok[s]
            if p % self.block_size == 0:
                need += 1
                continue
            b = self.tables[s][p // self.block_size]
            r = refs.get(b, self.ref[b])
            if r > 1:
                need += 1
                refs[b] = r - 1
        return need

    def append_slot(self, seq: int):
        """Reserve the slot of the next token of `seq`.

        Returns (slot, cow) where cow is None or (src, dst): the shared block
        src must be copied to the fresh block dst before the write."""
        return self.append_slots([seq])[0]

    def append_slots(self, seqs):
        """append_slot for each listed sequence in order; all or nothing."""
        if any(s in self.swapped for s in seqs):
            raise ValueError("a swapped-out sequence cannot be appended to")
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence may appear once per batch")
        need = self._blocks_for_appends(seqs)
        if need > len(self.free):
            raise OracleNoBlocks(f"need {need}, free {len(self.free)}")
        out = []
        bs = self.block_size
        for s in seqs:
            p = self.ntok[s]
            t = self.tables[s]
            lblk, off = p // bs, p % bs
            cow = None
            if off == 0:
                # the position starts a new logical block: take one now
                assert lblk == len(t)
                t.append(self._take())
            elif self.ref[t[lblk]] > 1:
                # writing into a shared block: duplicate it, then write
                src = t[lblk]
                dst = self._take()
                self.ref[src] -= 1
                t[lblk] = dst
                cow = (src, dst)
            self.ntok[s] = p + 1
            out.append((t[lblk] * bs + off, cow))
        return out

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent (partial last block
        included) and the parent's token count."""
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        if parent in self.swapped:
            raise ValueError("a swapped-out sequence cannot be forked")
        self.tables[child] = list(self.tables[parent])
        self.ntok[child] = self.ntok[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq: int) -> None:
        """Drop a sequence; blocks whose count reaches zero rejoin the back
        of the free list in table order. A swapped-out sequence returns its
        swap blocks instead."""
        t = self.tables[seq]
        if seq in self.swapped:
            self.swap_free.extend(t)
            self.swapped.discard(seq)
            del self.tables[seq]
            del self.ntok[seq]
            return
        for b in t:
            if self.ref[b] <= 0:
                raise OracleRefcountError(f"block {b}")
        for b in t:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[seq]
        del self.ntok[seq]

    # -- swapping ([N4N] "Why it matters for KV cache": under memory
    # pressure blocks are evicted to CPU memory and fetched back when the
    # request resumes; [ZQ] summary: easy preemption) ---------------------
    def set_swap_space(self, num_cpu_blocks: int) -> None:
        if self.swapped:
            raise ValueError("swap space in use")
        self.swap_free = deque(range(int(num_cpu_blocks)))

    def swap_out(self, seq: int):
        """Every table entry, in order, moves to the next free swap block;
        returns the (device block, swap block) moves. The device block is
        released once (it stays on the device while other sequences share
        it)."""
        if seq in self.swapped:
            raise ValueError("already swapped out")
        t = self.tables[seq]
        if len(t) > len(self.swap_free):
            raise OracleNoBlocks(f"need {len(t)} swap blocks, free {len(self.swap_free)}")
        moves = []
        for k, b in enumerate(t):
            c = self.swap_free.popleft()
            moves.append((b, c))
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
            t[k] = c
        self.swapped.add(seq)
        return moves

    def swap_in(self, seq: int):
        """Every swap block, in table order, gets a fresh device block from
        the front of the free list; returns the (swap block, device block)
        moves; the swap blocks rejoin the back of the swap free list."""
        if seq not in self.swapped:
            raise ValueError("not swapped out")
        t = self.tables[seq]
        if len(t) > len(self.free):
            raise OracleNoBlocks(f"need {len(t)}, free {len(self.free)}")
        moves = []
        for k, c in enumerate(t):
            d = self._take()
            moves.append((c, d))
            self.swap_free.append(c)
            t[k] = d
        self.swapped.discard(seq)
        return moves

    def export(self, seqs, max_blocks: int):
        """Block tables padded with -1 (the [N4N] BlockTable's "unallocated"
        marker) and token counts, for the listed sequences."""
        tab = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for r, s in enumerate(seqs):
            t = self.tables[s]
            if s in self.swapped:
                raise ValueError("a swapped-out sequence has no device table")
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            tab[r, :len(t)] = t
            lens[r] = self.ntok[s]
        return tab, lens


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of fp32 data or of bf16 bit patterns (uint16):
    a bf16 value is the upper half of the fp32 with the same bits."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x).view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def positions_to_rows(table, seq_len: int, block_size: int):
    """Per attended position p < seq_len: the physical block table[p // bs]
    and the offset p % bs inside it ([ZQ] pseudo-code, per-position
    dereference in the attention loop)."""
    pos = np.arange(int(seq_len))
    phys = np.asarray(table, dtype=np.int64)[pos // block_size]
    off = pos % block_size
    return phys, off


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: heads are grouped contiguously,
    h // (Hq / Hkv)."""
    return q_head // (num_q_heads // num_kv_heads)


def _gather(pool: np.ndarray, phys, off, kv_head: int) -> np.ndarray:
    return pool[phys, kv_head, off, :]


def _softmax_weighted_sum(scores: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Exact softmax of `scores` applied to the rows of `values`."""
    m = scores.max()
    w = np.exp(scores - m)
    return (w @ values) / w.sum()


def decode_one(q_row, k_pool, v_pool, table, seq_len, scale, kv_head, block_size):
    """Decode output of one query row (float64 [D]) attending to the first
    seq_len positions of one sequence through its block table."""
    d = k_pool.shape[-1]
    if seq_len == 0:
        return np.zeros(d, dtype=np.float64)
    phys, off = positions_to_rows(table, seq_len, block_size)
    keys = _gather(k_pool, phys, off, kv_head)
    vals = _gather(v_pool, phys, off, kv_head)
    scores = float(scale) * (keys @ q_row)
    return _softmax_weighted_sum(scores, vals)


def decode(q, k_pool, v_pool, block_tables, seq_lens, scale):
    """Paged decode attention, float64.

    q [B, Hq, D]; k_pool, v_pool [NB, Hkv, bs, D]; block_tables [B, maxb]
    (row i lists sequence i's physical blocks in logical order); seq_lens [B].
    Output [B, Hq, D]. [ZQ] pseudo-code and "Red flags" (the attention math
    is that of ordinary attention; only where K/V live changes); [Vij]
    "Borrow the abstraction" (logical order is kept, physical blocks are
    scattered)."""
    q = np.asarray(q, dtype=np.float64)
    B, hq, d = q.shape
    hkv, bs = k_pool.shape[1], k_pool.shape[2]
    out = np.zeros((B, hq, d), dtype=np.float64)
    for i in range(B):
        for h in range(hq):
            out[i, h] = decode_one(q[i, h], k_pool, v_pool, block_tables[i],
                                   int(seq_lens[i]), scale,
                                   kv_head_of(h, hq, hkv), bs)
    return out


def partition_partials(q_row, k_pool, v_pool, table, seq_len, scale, kv_head,
                       block_size, partition_tokens):
    """Split the context into partitions of `partition_tokens` positions and
    return, per partition j, (m_j, l_j, o_j): the max score, the sum of
    exp(score - m_j), and the partition's own normalised output."""
    parts = []
    for start in range(0, int(seq_len), int(partition_tokens)):
        stop = min(int(seq_len), start + int(partition_tokens))
        pos = np.arange(start, stop)
        phys = np.asarray(table, dtype=np.int64)[pos // block_size]
        off = pos % block_size
        keys = _gather(k_pool, phys, off, kv_head)
        vals = _gather(v_pool, phys, off, kv_head)
        s = float(scale) * (keys @ q_row)
        m = s.max()
        w = np.exp(s - m)
        parts.append((m, w.sum(), (w @ vals) / w.sum()))
    return parts


def combine_partials(parts, d):
    """Log-sum-exp combine: M = max m_j, weights l_j exp(m_j - M), output
    = sum_j weight_j o_j / sum_j weight_j."""
    if not parts:
        return np.zeros(d, dtype=np.float64)
    big_m = max(p[0] for p in parts)
    wts = np.array([p[1] * math.exp(p[0] - big_m) for p in parts])
    outs = np.stack([p[2] for p in parts])
    return (wts @ outs) / wts.sum()


def decode_partitioned(q, k_pool, v_pool, block_tables, seq_lens, scale,
                       partition_tokens):
    """decode() computed partition by partition and combined (must equal the
    unsplit result up to rounding)."""
    q = np.asarray(q, dtype=np.float64)
    B, hq, d = q.shape
    hkv, bs = k_pool.shape[1], k_pool.shape[2]
    out = np.zeros((B, hq, d), dtype=np.float64)
    for i in range(B):
        for h in range(hq):
            parts = partition_partials(q[i, h], k_pool, v_pool, block_tables[i],
                                       int(seq_lens[i]), scale,
                                       kv_head_of(h, hq, hkv), bs, partition_tokens)
            out[i, h] = combine_partials(parts, d)
    return out


def multi_query(q, k_pool, v_pool, block_tables, seq_lens, query_start, scale):
    """Attention of several query tokens per sequence over its paged cache,
    float64, causal inside the chunk.

    Sequence i's query tokens are rows query_start[i] .. query_start[i+1]-1
    of q [T, Hq, D]; they are its last Tq_i = query_start[i+1] -
    query_start[i] positions, already written to the cache, so seq_lens[i]
    counts them. Token t (0 <= t < Tq_i) sits at position L_i - Tq_i + t and
    attends to positions 0 .. L_i - Tq_i + t through the block table. Output
    [T, Hq, D].

    [ZQ] comparison table: paged attention is ordinary FlashAttention with a
    block-table dereference ("Real kernels fuse this with FlashAttention
    tiling", pseudo-code comment); the multi-token form is the reading taken
    for a prefill chunk or speculative tokens: standard causal attention
    whose key/value rows come through the table. With one query token per
    sequence it is exactly `decode`.
    """
    q = np.asarray(q, dtype=np.float64)
    T, hq, d = q.shape
    hkv = k_pool.shape[1]
    bs = k_pool.shape[2]
    out = np.zeros((T, hq, d), dtype=np.float64)
    starts = [int(x) for x in query_start]
    for i in range(len(starts) - 1):
        t0, t1 = starts[i], starts[i + 1]
        L = int(seq_lens[i])
        tq = t1 - t0
        if tq > L:
            raise ValueError("more query tokens than cached positions")
        for t in range(tq):
            n_att = L - tq + t + 1            # positions 0 .. L - tq + t
            for h in range(hq):
                g = kv_head_of(h, hq, hkv)
                out[t0 + t, h] = decode_one(q[t0 + t, h], k_pool, v_pool, block_tables[i],
                                            n_att, scale, g, bs)
    return out


# --------------------------------------------------------------------------
# Cache writes
# --------------------------------------------------------------------------

def reshape_and_cache(k_new, v_new, slot_mapping, k_pool, v_pool):
    """Write token t's K and V rows (every KV head) into slot slot_mapping[t]
    = block * bs + offset of the pools, bit for bit; slot < 0 writes nothing.
    In place on numpy arrays of any element type. [ZQ] pseudo-code: the new
    token's K/V go to the last block at offset pos % bs; [ZQ] comparison
    table: generation writes into the current block."""
    bs = k_pool.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, o = slot // bs, slot % bs
        k_pool[b, :, o, :] = k_new[t]
        v_pool[b, :, o, :] = v_new[t]


def copy_blocks(k_pool, v_pool, pairs):
    """For each (src, dst): both pools' block dst becomes a bit copy of block
    src. [FP] "Copy-on-write sharing": the diverging sequence gets a copy of
    the one shared block before it writes."""
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """For each (src, dst): block dst of the destination pools becomes a bit
    copy of block src of the source pools (device pools to swap space or
    back; [N4N] "Why it matters for KV cache", swapping and preemption)."""
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]


# --------------------------------------------------------------------------
# 8-bit KV pool (FP8 E4M3, OCP definition)
# --------------------------------------------------------------------------
# [ZQ] summary: paged attention composes with KV quantization; the pages give
# no scheme. Reading taken: OCP FP8 E4M3 ("fn": no infinities, S.1111.111 is
# NaN, largest finite 448), one float32 scale per pool (K and V); a value x is
# stored as the code nearest to the exact quotient x / scale (ties to the code
# with an even mantissa), saturating to +-448; the code's value times the
# scale is what attention reads.

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one FP8 E4M3 code: sign, 4-bit exponent (bias 7), 3-bit
    mantissa; exponent 0 holds the subnormals m * 2^-9; S.1111.111 is NaN."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_values(codes) -> np.ndarray:
    """Float64 values of an array of codes (uint8)."""
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def _nearest_code(y) -> np.ndarray:
    """Nearest FP8 E4M3 code to each float64 value of y (ties to the code with
    an even mantissa), saturating at +-448; NaN gives 0x7F with y's sign.
    Written as a search over the 127 non-negative finite codes."""
    y = np.asarray(y, dtype=np.float64)
    mags = np.array([e4m3_value(c) for c in range(0x7F)])        # codes 0x00..0x7E, ascending
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)  # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)
    code = np.where(np.isnan(y), np.where(np.signbit(y), 0xFF, 0x7F), code).astype(np.uint8)
    return code


def e4m3_encode(x) -> np.ndarray:
    """Nearest FP8 E4M3 code to each float32 value of x (ties to the code with
    an even mantissa), saturating at +-448; NaN gives 0x7F with the input's
    sign."""
    return _nearest_code(np.asarray(x, dtype=np.float32).astype(np.float64))


def quantize_e4m3(x, scale: float) -> np.ndarray:
    """Codes of x / scale: the code nearest to the exact quotient of each
    float32 value of x (e.g. from bf16) by the float32 scale.

    The quotient is formed in float64. That decides every case as the exact
    quotient would: a midpoint between two codes has at most 5 significant
    bits, so the exact quotient x / s of two float32 values is either that
    midpoint exactly (a tie) or differs from it by at least 2^-29 of its
    size, far more than the 2^-53 of one float64 rounding; the rounded
    quotient therefore lies on the same side of every midpoint."""
    q = (np.asarray(x, dtype=np.float32).astype(np.float64) /
         np.float64(np.float32(scale)))
    return _nearest_code(q)


def reshape_and_cache_e4m3(k_new, v_new, slot_mapping, k_codes, v_codes, k_scale, v_scale):
    """The slot write into 8-bit pools: token t's K and V rows (float32
    values) are quantized with their pool's scale and stored at slot
    slot_mapping[t] = block * bs + offset; slot < 0 writes nothing."""
    bs = k_codes.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, o = slot // bs, slot % bs
        k_codes[b, :, o, :] = quantize_e4m3(k_new[t], k_scale)
        v_codes[b, :, o, :] = quantize_e4m3(v_new[t], v_scale)


def dequantize_e4m3(codes, scale: float) -> np.ndarray:
    """What attention reads from an 8-bit pool: code value times the scale
    (float64; the scale is taken as its float32 value)."""
    return e4m3_values(codes) * float(np.float32(scale))
