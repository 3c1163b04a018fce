"""GPU parity on very long contexts: sequences of 200,000 and 65,537 positions
beside short ones, every output row against the plain-C float64 oracle.

These lengths reach code the usual workloads do not: block-table windows
re-read hundreds of times by one wave (unsplit walks), thousands of
partitions per row for the merge, the automatic 1024-position partitions of
long contexts, and a work plan whose last partitions range from 1 to 1024
positions. The multi-token tiled kernel walks a 12,000-position context."""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import bench_step, build, check_close, to_device, to_storage_np

pytestmark = pytest.mark.gpu

VALU, MFMA = P.PA_VARIANT_VALU, P.PA_VARIANT_MFMA
LONG_LENS = [1, 200_000, 65_537, 3_000]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


@pytest.fixture(scope="module")
def long_case(dev):
    w = W.Workload("long", 601, 0, 32, 8, 128, 16, "bf16", ("fixed", 0), ("factor", 1.1))
    return build(w, dev, lens=LONG_LENS, pool_on_device=True, append=False)


def _f64(t):
    return O.as_f64(to_storage_np(t), "bf16")


@pytest.fixture(scope="module")
def long_ref(long_case):
    return long_case.oracle_c()


# 0: automatic partitions (1024 positions beyond 8192); 64: 3,125 partitions
# for the longest row; -1: unsplit (one workgroup walks the whole context)
@pytest.mark.parametrize("ptok", [0, 64, -1])
@pytest.mark.parametrize("variant", [MFMA, VALU])
def test_long_decode_every_row(dev, long_case, long_ref, variant, ptok):
    out = long_case.decode(variant=variant, partition_tokens=ptok)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    err = check_close(_f64(out), long_ref, "bf16", f"long decode variant {variant} ptok {ptok}")
    print(f"long decode variant {variant} ptok {ptok}: max_abs {err[0]:.3g} max_rel {err[1]:.3g}",
          flush=True)


def test_long_planned_step(dev):
    # the bench's launch (slot write, partition kernel over a work plan,
    # merge) on its own case: the step appends one token to every sequence
    w = W.Workload("long_step", 603, 0, 32, 8, 128, 16, "bf16", ("fixed", 0), ("factor", 1.1))
    # table rows wide enough for the appended token (200,000 + 1 starts a block)
    maxb = max(O.blocks_needed(L + 1, 16) for L in LONG_LENS)
    c = build(w, dev, lens=LONG_LENS, pool_on_device=True, append=False, max_blocks=maxb)
    out = bench_step(c, seed=5)
    assert c.olens.tolist() == [L + 1 for L in LONG_LENS]
    check_close(_f64(out), c.oracle_c(), "bf16", "long planned step")


def test_long_context_tiled_multi_query(dev):
    lens, tqs = [12_000, 3_000], [40, 33]
    w = W.Workload("long_mq", 605, 0, 32, 8, 128, 16, "bf16", ("fixed", 0), ("factor", 1.2))
    c = build(w, dev, lens=lens, append=False)
    rng = np.random.default_rng(606)
    qs = np.concatenate([[0], np.cumsum(tqs)]).astype(np.int32)
    q_np = W.normal_values((int(qs[-1]), 32, 128), rng, "bf16")
    out = torch.full((int(qs[-1]), 32, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    P.pa_multi_query(to_device(q_np, "bf16", dev), c.k_pool, c.v_pool, c.tables, c.lens,
                     torch.from_numpy(qs).to(dev), c.scale, out, max_seq_len=c.max_len,
                     max_query_len=max(tqs))
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    ref = O.multi_query(O.as_f64(q_np, "bf16"), O.as_f64(c.ok_pool, "bf16"),
                        O.as_f64(c.ov_pool, "bf16"), c.otables, c.olens, qs, c.scale)
    check_close(_f64(out), ref, "bf16", "long-context tiled multi-query")
