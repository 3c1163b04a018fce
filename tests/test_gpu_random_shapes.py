"""Randomized GPU parity sweep: decode, multi-token and shared-prefix calls on
seeded random shapes (heads, group, block size, partition length, lengths
with the edge values mixed in) against the float64 oracle, every output."""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import build, check_close, scale_for, to_device, to_storage_np

pytestmark = pytest.mark.gpu

EDGE = [0, 1, 15, 16, 17, 255, 256, 257, 511, 512, 513]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _draw_shape(rng):
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    bs = int(rng.choice([16, 32, 64, 128]))
    B = int(rng.integers(1, 12))
    lens = [int(x) for x in rng.choice(EDGE + list(rng.integers(1, 1500, 8)), size=B)]
    ptok = int(rng.choice([0, -1, bs, 2 * bs, 256, 512]))
    if ptok > 0 and ptok % bs:
        ptok = 0
    return hkv * group, hkv, bs, lens, ptok


@pytest.mark.parametrize("case", range(24))
def test_random_decode(dev, case):
    rng = np.random.default_rng(9000 + case)
    hq, hkv, bs, lens, ptok = _draw_shape(rng)
    w = W.Workload("rand", 9000 + case, 0, hq, hkv, 128, bs, "bf16", ("fixed", 0), ("factor", 1.2))
    c = build(w, dev, lens=lens, append=False)
    out = c.decode(partition_tokens=ptok)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    check_close(O.as_f64(to_storage_np(out), "bf16"), c.oracle_all(), "bf16",
                f"decode hq {hq} hkv {hkv} bs {bs} ptok {ptok} lens {lens}")
    # the same decode over a host work plan: bit-identical
    shape = P._decode_shape(c.q, c.k_pool, c.tables, c.max_len, ptok, P.PA_VARIANT_AUTO)
    plan_np = P.pa_decode_plan(shape, c.olens)
    out_p = torch.full_like(out, float("nan"))
    P.pa_decode(c.q, c.k_pool, c.v_pool, c.tables, c.lens, c.scale, out_p,
                        work_plan=torch.from_numpy(plan_np).to(dev), max_seq_len=c.max_len,
                        partition_tokens=ptok)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    assert torch.equal(out_p.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("case", range(12))
def test_random_multi_query(dev, case):
    rng = np.random.default_rng(9100 + case)
    hq, hkv, bs, lens, _ = _draw_shape(rng)
    lens = [max(1, L) for L in lens]
    tqs = [int(rng.integers(0, min(L, 80) + 1)) for L in lens]
    split = bool(rng.integers(0, 2))
    ptok = int(rng.choice([0, 16, 64, 256]))
    w = W.Workload("randmq", 9100 + case, 0, hq, hkv, 128, bs, "bf16", ("fixed", 0),
                   ("factor", 1.2))
    c = build(w, dev, lens=lens, append=False)
    qs = np.concatenate([[0], np.cumsum(tqs)]).astype(np.int32)
    T = max(1, int(qs[-1]))
    q_np = W.normal_values((T, hq, 128), rng, "bf16")
    out = torch.zeros((T, hq, 128), dtype=torch.bfloat16, device=dev)
    P.pa_multi_query(to_device(q_np, "bf16", dev), c.k_pool, c.v_pool, c.tables, c.lens,
                     torch.from_numpy(qs).to(dev), c.scale, out, max_seq_len=c.max_len,
                     max_query_len=max(1, max(tqs)), split=split, partition_tokens=ptok)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    ref = O.multi_query(O.as_f64(q_np, "bf16"), O.as_f64(c.ok_pool, "bf16"),
                        O.as_f64(c.ov_pool, "bf16"), c.otables, c.olens, qs, c.scale)
    got = O.as_f64(to_storage_np(out), "bf16")
    check_close(got[:int(qs[-1])], ref[:int(qs[-1])], "bf16",
                f"mq hq {hq} hkv {hkv} bs {bs} split {split} ptok {ptok} lens {lens} tqs {tqs}")
