"""GPU parity of the matrix-core decode kernel on shapes whose full grid
(sequences x KV heads x partitions) has 1024 or more workgroups, where it
runs with 2 waves per workgroup (smaller grids take 4):
every block size, 1 and 4 query heads per KV head, bf16 and 8-bit pools,
planned and unplanned. Every output element is compared with the plain-C
float64 oracle; planned and unplanned results must agree bit for bit."""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import build, check_close, to_device, to_storage_np

pytestmark = pytest.mark.gpu

MFMA = P.PA_VARIANT_MFMA


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _lens(n, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 1100, n)
    lens[:8] = [0, 1, 15, 16, 17, 512, 513, 1099]
    return lens.tolist()


@pytest.mark.parametrize("bs", [8, 16, 32, 64, 128])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8)])
def test_bf16_wide_grid(dev, bs, hq, hkv):
    w = W.Workload("wide", 171, 0, hq, hkv, 128, bs, "bf16", ("fixed", 0), ("factor", 1.1))
    c = build(w, dev, lens=_lens(160, 171 + bs), append=False, pool_on_device=True)
    print("wide bf16", bs, hq, hkv, flush=True)
    shape = P._decode_shape(c.q, c.k_pool, c.tables, c.max_len, 0, MFMA)
    assert c.B * c.hkv * -(-c.max_len // 512) >= 1024
    out = c.decode(variant=MFMA)
    plan = torch.from_numpy(P.pa_decode_plan(shape, c.olens)).to(dev)
    out_p = torch.empty_like(out)
    P.pa_decode(c.q, c.k_pool, c.v_pool, c.tables, c.lens, c.scale, out_p,
                        work_plan=plan, max_seq_len=c.max_len, variant=MFMA)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    assert torch.equal(out.view(torch.int16), out_p.view(torch.int16))
    got_all = O.as_f64(to_storage_np(out), "bf16")
    check_close(got_all, c.oracle_c(), "bf16", f"wide bf16 bs {bs} {hq}/{hkv}")
    assert not got_all[0].any()


@pytest.mark.parametrize("bs", [16, 64])
def test_e4m3_wide_grid(dev, bs):
    w = W.Workload("wide8", 181, 0, 32, 8, 128, bs, "bf16", ("fixed", 0), ("factor", 1.1))
    c = build(w, dev, lens=_lens(160, 181 + bs), append=False)
    print("wide e4m3", bs, flush=True)
    rng = np.random.default_rng(182)
    kc = W.random_e4m3_codes((c.nb, c.hkv, bs, 128), rng)
    vc = W.random_e4m3_codes((c.nb, c.hkv, bs, 128), rng)
    kc_t, vc_t = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    # every finite code of both signs reaches the decode: q / 16 (exact)
    # keeps the scores over codes up to 448 x k_scale a few units wide
    c.oq = W.to_bf16_bits((O.as_f64(c.oq, "bf16") / 16).astype(np.float32))
    c.q = to_device(c.oq, "bf16", dev)
    ks, vs = 0.37, 0.11
    outs = []
    shape = P._decode_shape(c.q, kc_t, c.tables, c.max_len, 512, MFMA)
    plan = torch.from_numpy(P.pa_decode_plan(shape, c.olens)).to(dev)
    assert c.B * c.hkv * -(-c.max_len // 512) >= 1024
    for wp in (None, plan):
        out = torch.empty_like(c.q)
        P.pa_decode_e4m3(c.q, kc_t, vc_t, c.tables, c.lens, c.scale, ks, vs, out,
                         max_seq_len=c.max_len, partition_tokens=512, work_plan=wp)
        outs.append(out)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    got_all = O.as_f64(to_storage_np(outs[0]), "bf16")
    check_close(got_all, c.oracle_c_e4m3(kc, vc, ks, vs), "bf16", f"wide e4m3 bs {bs}")
