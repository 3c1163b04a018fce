"""GPU parity of the planned decode (pa_decode_plan, then pa_decode or
pa_decode_partition with the work_plan argument): each work unit computes what it computes in
pa_decode, so outputs must be bitwise equal to pa_decode's, and within
tolerance of the float64 oracle; bad plan entries are skipped and flagged."""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import build, check_close, to_storage_np

pytestmark = pytest.mark.gpu

VALU, MFMA = P.PA_VARIANT_VALU, P.PA_VARIANT_MFMA


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _custom(name, seed, hq, hkv, d, bs, dtype):
    return W.Workload(name, seed, 0, hq, hkv, d, bs, dtype, ("fixed", 0), ("factor", 1.3))


def _planned(c, variant=P.PA_VARIANT_AUTO, ptok=0, split=False):
    shape = P._decode_shape(c.q, c.k_pool, c.tables, c.max_len, ptok, variant)
    plan = torch.from_numpy(P.pa_decode_plan(shape, c.olens)).to(c.device)
    out = torch.empty_like(c.q)
    kw = dict(work_plan=plan, max_seq_len=c.max_len, partition_tokens=ptok, variant=variant)
    if split:
        ws = torch.empty(max(P.pa_decode_workspace_bytes(shape), 16), dtype=torch.uint8,
                         device=c.device)
        P.pa_decode_partition(c.q, c.k_pool, c.v_pool, c.tables, c.lens, c.scale, out,
                                      workspace=ws, **kw)
        P.pa_decode_reduce(c.q, c.k_pool, c.tables, c.lens, out, max_seq_len=c.max_len,
                           partition_tokens=ptok, variant=variant, workspace=ws)
    else:
        P.pa_decode(c.q, c.k_pool, c.v_pool, c.tables, c.lens, c.scale, out, **kw)
    return out


EDGE_LENS = [0, 1, 15, 16, 17, 511, 512, 513, 1024, 1025, 1537, 0, 3]

SHAPES = [
    # dtype, hq, hkv, d, bs, variant
    ("bf16", 32, 8, 128, 16, MFMA),
    ("bf16", 32, 8, 128, 16, VALU),
    ("bf16", 16, 16, 128, 32, MFMA),     # two blocks of 8 KV heads per round
    ("bf16", 40, 40, 128, 16, MFMA),     # Hkv 40: five head blocks
    ("bf16", 8, 4, 128, 16, MFMA),       # Hkv not a multiple of 8
    ("bf16", 32, 8, 128, 8, MFMA),
    ("bf16", 32, 8, 128, 128, MFMA),
    ("bf16", 64, 8, 128, 16, VALU),      # group 8 on the vector kernel
    ("bf16", 64, 8, 128, 16, MFMA),      # group 8: the multi-token per-tile kernel
    ("bf16", 16, 1, 128, 32, MFMA),      # group 16: the same, one tile per token
    ("f32", 8, 2, 128, 32, VALU),
    ("f32", 4, 4, 64, 16, VALU),
]


@pytest.mark.parametrize("ptok", [0, 16, 64])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_planned_equals_unplanned_and_oracle(dev, shape, ptok):
    dtype, hq, hkv, d, bs, variant = shape
    if ptok and ptok % bs:
        pytest.skip("partition length must be a multiple of the block size")
    w = _custom("planned", 131, hq, hkv, d, bs, dtype)
    c = build(w, dev, lens=EDGE_LENS, append=False)
    print("planned", shape, ptok, flush=True)
    ref_out = c.decode(variant=variant, partition_tokens=ptok)
    for split in (False, True):
        out = _planned(c, variant, ptok, split)
        torch.cuda.synchronize()
        assert P.pa_device_errors() == 0
        assert torch.equal(out.view(torch.int16) if dtype == "bf16" else out.view(torch.int32),
                           ref_out.view(torch.int16) if dtype == "bf16" else
                           ref_out.view(torch.int32)), f"planned != pa_decode ({shape}, split={split})"
    got = O.as_f64(to_storage_np(out), dtype)
    check_close(got, c.oracle_all(), dtype, f"planned {shape} ptok {ptok}")
    assert not got[0].any() and not got[11].any()          # empty sequences give zeros


@pytest.mark.parametrize("name", ["llama3_8b", "llama2_13b"])
def test_planned_full_size_bitwise(dev, name):
    """The workloads at full size in the bench's launch configuration: the
    planned partition kernel + merge equals pa_decode bitwise on every output
    (pa_decode itself is checked against the oracle at full size in
    test_gpu_workloads.py)."""
    w = W.get(name)
    c = build(w, dev, pool_on_device=True)
    print("planned full size", name, flush=True)
    ref_out = c.decode()
    out = _planned(c, split=True)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))


def test_planned_e4m3_full_size_bitwise(dev):
    """The headline shape over 8-bit pools (the bench's --kv-dtype e4m3 leg:
    partitions of 1024 positions): planned = unplanned bitwise."""
    w = W.get("llama3_8b")
    c = build(w, dev, pool_on_device=True)
    print("planned full size e4m3", flush=True)
    kc = W.random_e4m3_codes_device(tuple(c.k_pool.shape), 901, dev)
    vc = W.random_e4m3_codes_device(tuple(c.v_pool.shape), 902, dev)
    shape = P._decode_shape(c.q, kc, c.tables, c.max_len, 1024, P.PA_VARIANT_MFMA)
    plan = torch.from_numpy(P.pa_decode_plan(shape, c.olens)).to(dev)
    outs = []
    for wp in (None, plan):
        out = torch.empty_like(c.q)
        P.pa_decode_e4m3(c.q, kc, vc, c.tables, c.lens, c.scale, 0.05, 0.05, out,
                         max_seq_len=c.max_len, partition_tokens=1024, work_plan=wp)
        outs.append(out)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("hq", [32, 64])
def test_bad_plan_entries_are_skipped_and_flagged(dev, hq):
    w = _custom("badplan", 132, hq, 8, 128, 16, "bf16")
    c = build(w, dev, lens=[40, 700], append=False)
    shape = P._decode_shape(c.q, c.k_pool, c.tables, c.max_len, 0, MFMA)
    plan = P.pa_decode_plan(shape, c.olens)
    # group 4: 512-position partitions (700 -> 2); group 8: 1024 (one each)
    assert plan.shape == ((3, 4) if hq == 32 else (2, 4))
    P.pa_device_errors()
    # sequence out of range, negative partition, a partition past the
    # sequence's last, a negative length, a length above the table's bound
    for bad in ([2, 0, 40, 0], [-1, 0, 40, 0], [1, 2, 700, 0], [0, -5, 40, 0],
                [0, 1, 40, 0], [0, 0, -3, 0], [1, 0, 10 ** 6, 0]):
        p = plan.copy()
        p[1] = bad                                   # replaces one valid unit
        pt = torch.from_numpy(p).to(dev)
        out = torch.zeros_like(c.q)
        P.pa_decode(c.q, c.k_pool, c.v_pool, c.tables, c.lens, c.scale, out,
                            work_plan=pt, max_seq_len=c.max_len, variant=MFMA)
        torch.cuda.synchronize()
        assert P.pa_device_errors() == P.PA_DEVERR_PLAN, bad
