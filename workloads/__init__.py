"""Seeded synthetic inputs for paged decode attention.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests. It only *draws* inputs: sequence lengths, the order in which the free
pool hands out physical blocks, and N(0,1) tensor contents. It holds none of
the method's arithmetic: block tables, slots, copy-on-write decisions and
attention are computed separately by each side from these draws.

The five workload shapes:

  single_fp32   1 sequence, 33 cached tokens, block size 16, 1/1 heads,
                head dim 64, fp32, 16-block pool (the 33-token allocation
                example of "PagedAttention Explained", "Grow allocation with
                the sequence").
  small_mha     8 sequences, pre-append lengths U{1..512}, 8/8 heads, D 128,
                block size 16, bf16, 512-block pool.
  llama2_13b    128 chat requests, prompt U{100..2000} + generated U{50..500}
                tokens, 40/40 heads, D 128, block size 16, bf16; pool = 1.2x
                the blocks the batch occupies (request mix of the chat-workload
                example on the n4n.ai page "What is PagedAttention ...").
  llama3_8b     256 sequences, lengths U{512..4096}, 32 query / 8 KV heads,
                D 128, block size 16, bf16, partitions of 512 tokens; pool =
                1.1x the occupied blocks.
  shared_prefix 64 prompt groups x 4 samples, 32/8 heads, D 128, block size
                32, bf16; each group's prompt (1040 tokens: 32 full blocks and
                one half-filled block) is shared by its 4 samples, then each
                sample appends a private suffix of U{16..256} tokens.
                The long variant adds 16 sequences of 32768 tokens. No
                partition length is fixed for these two (partition_tokens 0:
                the library's automatic choice).

Draw order for every workload (one numpy Generator seeded with the workload's
seed): lengths -> free-list order -> q -> new k/v -> pool contents.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "draw_lengths", "pool_blocks",
    "free_order", "normal_f32", "to_bf16_bits", "normal_values", "random_e4m3_codes",
]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f32" or "bf16"
    lengths: tuple                  # recipe, see draw_lengths()
    pool: tuple                     # ("fixed", NB) or ("factor", f)
    partition_tokens: int = 512
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "single_fp32": Workload("single_fp32", 1, 1, 1, 1, 64, 16, "f32",
                            ("fixed", 33), ("fixed", 16)),
    "small_mha": Workload("small_mha", 2, 8, 8, 8, 128, 16, "bf16",
                          ("uniform", 1, 512), ("fixed", 512)),
    "llama2_13b": Workload("llama2_13b", 3, 128, 40, 40, 128, 16, "bf16",
                           ("sum_uniform", (100, 2000), (50, 500)), ("factor", 1.2)),
    "llama3_8b": Workload("llama3_8b", 4, 256, 32, 8, 128, 16, "bf16",
                          ("uniform", 512, 4096), ("factor", 1.1)),
    "shared_prefix": Workload("shared_prefix", 5, 256, 32, 8, 128, 32, "bf16",
                              ("prefix_suffix", 1040, (16, 256), 4), ("factor", 1.1),
                              partition_tokens=0, extra={"groups": 64, "samples": 4}),
    "shared_prefix_long": Workload("shared_prefix_long", 5, 272, 32, 8, 128, 32, "bf16",
                                   ("prefix_suffix", 1040, (16, 256), 4), ("factor", 1.1),
                                   partition_tokens=0,
                                   extra={"groups": 64, "samples": 4,
                                          "long_seqs": 16, "long_len": 32768}),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def draw_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    """Per-sequence token counts (int64) drawn per the workload's recipe.

    For "prefix_suffix" the result is the private suffix length per sample
    (the shared prompt length is w.lengths[1]); for the long variant the 16
    long sequences follow the 256 samples and carry their full length.
    """
    kind = w.lengths[0]
    if kind == "fixed":
        return np.full(w.num_seqs, w.lengths[1], dtype=np.int64)
    if kind == "uniform":
        lo, hi = w.lengths[1], w.lengths[2]
        return rng.integers(lo, hi + 1, size=w.num_seqs, dtype=np.int64)
    if kind == "sum_uniform":
        (a0, a1), (b0, b1) = w.lengths[1], w.lengths[2]
        prompt = rng.integers(a0, a1 + 1, size=w.num_seqs, dtype=np.int64)
        gen = rng.integers(b0, b1 + 1, size=w.num_seqs, dtype=np.int64)
        return prompt + gen
    if kind == "prefix_suffix":
        s0, s1 = w.lengths[2]
        n_samples = w.extra["groups"] * w.extra["samples"]
        suffix = rng.integers(s0, s1 + 1, size=n_samples, dtype=np.int64)
        if "long_seqs" in w.extra:
            suffix = np.concatenate(
                [suffix, np.full(w.extra["long_seqs"], w.extra["long_len"], dtype=np.int64)])
        return suffix
    raise ValueError(kind)


def pool_blocks(w: Workload, occupied_blocks: int) -> int:
    """Physical pool size for a workload whose sequences occupy
    `occupied_blocks` blocks (the caller counts them): a fixed size, or the
    stated over-provisioning factor on top of the occupied count."""
    kind = w.pool[0]
    if kind == "fixed":
        return int(w.pool[1])
    return int(math.ceil(w.pool[1] * occupied_blocks))


def free_order(num_blocks: int, rng: np.random.Generator) -> np.ndarray:
    """Order in which the free pool hands out physical block ids: a seeded
    permutation of range(num_blocks) (int32)."""
    return rng.permutation(num_blocks).astype(np.int32)


def normal_f32(shape, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 by round-to-nearest-even, returned as uint16 bit patterns.
    (Input preparation: the rounding of a draw into the storage type.)"""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_values(shape, rng: np.random.Generator, dtype: str) -> np.ndarray:
    """N(0,1) draws in the storage type: float32 array, or uint16 bf16 bits."""
    x = normal_f32(shape, rng)
    return x if dtype == "f32" else to_bf16_bits(x)


def random_e4m3_codes(shape, rng: np.random.Generator) -> np.ndarray:
    """Random FP8 E4M3 bytes for an 8-bit pool: every finite code point of
    either sign (0x00..0x7E, then a random sign bit), drawn uniformly over
    code points. Raw bytes; the format's arithmetic is not used here."""
    low = rng.integers(0, 0x7F, size=shape, dtype=np.uint8)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    return (low | sign).astype(np.uint8)


def random_e4m3_codes_device(shape, seed: int, device):
    """random_e4m3_codes drawn on `device` by torch's seeded generator (uint8
    tensor), for pools too large to draw on the host quickly."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    low = torch.randint(0, 0x7F, tuple(shape), generator=g, device=device, dtype=torch.int32)
    sign = torch.randint(0, 2, tuple(shape), generator=g, device=device, dtype=torch.int32)
    return (low | (sign << 7)).to(torch.uint8)


def normal_device(shape, seed: int, dtype: str, device):
    """N(0,1) draws made on `device` by torch's seeded generator (used for
    pools too large to draw on the host quickly). Returns a torch tensor of
    float32 or bfloat16; the same seed gives the same values on one device."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return t if dtype == "f32" else t.to(torch.bfloat16)
