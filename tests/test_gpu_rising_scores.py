"""Scores that rise along the context, so that every softmax stream keeps
moving its reference maximum: the kernels move a stream's reference only when
a score passes it by more than 2^8 (log2 units) and skip the output rescale
while no stream of the wave moved. Key dimension 0 of position p carries
`slope * p` and the query's dimension 0 a constant, so the score grows by a
fixed step per position:

- steep: about 1.5 (log2 units) per position, 24 per 16-position chunk: the
  reference moves at every chunk and the output is dominated by the last few
  positions;
- gentle: about 0.25 per position, 4 per chunk: the reference moves every
  second chunk or so, and exponents up to 2^8 pile up in between.

Decode at 1, 4 and 8 query heads per KV head (the decode kernel and the
per-tile kernel, split partitions and not), decode over 8-bit pools, and
multi-token chunks (the per-tile and the workgroup-tiled kernels) against the
float64 oracle under
the bf16 tolerance. The math is ordinary attention ("Walk through paged
attention end to end ...", single-decode-step pseudo-code and "Red flags")."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import build, check_close, to_device, to_storage_np

pytestmark = pytest.mark.gpu

# score step per position in log2 units: steep and gentle ramps
RAMPS = {"steep": 1.5, "gentle": 0.25}
Q0 = 4.0          # the query's dimension 0


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _ramp_case(dev, hq, hkv, bs, lens, step, seed):
    """A case whose K rows carry slope * p in dimension 0 (small noise
    elsewhere) and whose queries carry Q0 there, so that the score of
    position p is about step * p in log2 units."""
    w = W.Workload("ramp", seed, 0, hq, hkv, 128, bs, "bf16", ("fixed", 0), ("factor", 1.2))
    c = build(w, dev, lens=lens, append=False)
    slope = step / (Q0 * c.scale * math.log2(math.e))
    kp = O.as_f64(c.ok_pool, "bf16").astype(np.float32) * 0.1
    for i, L in enumerate(c.olens):
        phys, off = O.positions_to_rows(c.otables[i], int(L), bs)
        kp[phys, :, off, 0] = (slope * np.arange(int(L)))[:, None]
    c.ok_pool = W.to_bf16_bits(kp)
    c.k_pool.copy_(to_device(c.ok_pool, "bf16", dev))
    return c


def _ramp_queries(shape, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape).astype(np.float32) * 0.1
    q[..., 0] = Q0
    return W.to_bf16_bits(q)


@pytest.mark.parametrize("ramp", sorted(RAMPS))
@pytest.mark.parametrize("hq,hkv,ptok", [(32, 8, 0), (32, 8, -1), (8, 8, 0), (64, 8, 0),
                                         (64, 8, -1)])
def test_decode_rising_scores(dev, ramp, hq, hkv, ptok):
    lens = [1, 17, 300, 513, 1100, 2048]
    c = _ramp_case(dev, hq, hkv, 16, lens, RAMPS[ramp], 401)
    c.oq = _ramp_queries((len(lens), hq, 128), 402)
    c.q = to_device(c.oq, "bf16", dev)
    out = torch.full_like(c.q, float("nan"))
    P.pa_decode(c.q, c.k_pool, c.v_pool, c.tables, c.lens, c.scale, out, max_seq_len=c.max_len,
                partition_tokens=ptok, variant=P.PA_VARIANT_MFMA)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    got = O.as_f64(to_storage_np(out), "bf16")
    assert np.isfinite(got).all()
    check_close(got, c.oracle_all(), "bf16", f"decode {ramp} {hq}/{hkv} ptok {ptok}")


@pytest.mark.parametrize("ramp", sorted(RAMPS))
@pytest.mark.parametrize("hq,hkv,tq,split", [(32, 8, 4, False), (32, 8, 4, True),
                                             (32, 8, 160, False)])
def test_multi_query_rising_scores(dev, ramp, hq, hkv, tq, split):
    """4 tokens per sequence on the per-tile kernel (split contexts and not),
    160 on the workgroup-tiled kernel (640 rows per KV head)."""
    lens = [700, 1500, 2100]
    c = _ramp_case(dev, hq, hkv, 16, lens, RAMPS[ramp], 411)
    tqs = [tq] * len(lens)
    qs = np.concatenate([[0], np.cumsum(tqs)]).astype(np.int32)
    q_np = _ramp_queries((int(qs[-1]), hq, 128), 412)
    q = to_device(q_np, "bf16", dev)
    out = torch.full((int(qs[-1]), hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    P.pa_multi_query(q, c.k_pool, c.v_pool, c.tables, c.lens, torch.from_numpy(qs).to(dev),
                     c.scale, out, max_seq_len=c.max_len, max_query_len=tq, split=split)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    ref = O.multi_query(O.as_f64(q_np, "bf16"), O.as_f64(c.ok_pool, "bf16"),
                        O.as_f64(c.ov_pool, "bf16"), c.otables, c.olens, qs, c.scale)
    got = O.as_f64(to_storage_np(out), "bf16")
    assert np.isfinite(got).all()
    check_close(got, ref, "bf16", f"multi-query {ramp} tq {tq} split {split}")


@pytest.mark.parametrize("ramp", sorted(RAMPS))
def test_decode_e4m3_rising_scores(dev, ramp):
    """The same over 8-bit pools: key dimension 0 holds the E4M3 code of
    slope * p / k_scale (the oracle's quantizer; other dimensions small random
    codes), so the scores climb in the format's coarse steps."""
    hq, hkv, bs, lens = 32, 8, 16, [1, 17, 300, 513, 1100, 2048]
    c = _ramp_case(dev, hq, hkv, bs, lens, RAMPS[ramp], 421)
    c.oq = _ramp_queries((len(lens), hq, 128), 422)
    c.q = to_device(c.oq, "bf16", dev)
    rng = np.random.default_rng(423)
    ks, vs = 16.0, 0.11
    kc = O.quantize_e4m3(O.as_f64(c.ok_pool, "bf16").astype(np.float32), ks)
    vc = W.random_e4m3_codes((c.nb, hkv, bs, 128), rng)
    # the slope's codes in dimension 0 (max 448 * 16 = 7168), small codes elsewhere
    small = W.random_e4m3_codes((c.nb, hkv, bs, 128), rng) & np.uint8(0x9F)
    kc[..., 1:] = small[..., 1:]
    out = torch.full_like(c.q, float("nan"))
    P.pa_decode_e4m3(c.q, torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev), c.tables,
                     c.lens, c.scale, ks, vs, out, max_seq_len=c.max_len)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    ref = O.decode(O.as_f64(c.oq, "bf16"), O.dequantize_e4m3(kc, ks), O.dequantize_e4m3(vc, vs),
                   c.otables, c.olens, c.scale)
    got = O.as_f64(to_storage_np(out), "bf16")
    assert np.isfinite(got).all()
    check_close(got, ref, "bf16", f"e4m3 decode {ramp}")
