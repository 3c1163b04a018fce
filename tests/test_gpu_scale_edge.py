"""GPU parity at softmax scales other than the usual positive 1/sqrt(D).

The calls accept any finite scale. A negative one makes the smallest dot
product the heaviest weight (the kernels fold its sign into q, so the scale
they apply to the scores is never negative); zero makes every visible
position weigh the same, so each output row is the plain mean of its V rows.
Every kernel family is compared element by element with the float64 oracle
(pinned to torch SDPA at negative scales and to the mean at scale 0): the
decode kernels (matrix-core, vector ALU, the per-tile kernel at 8 query
heads per KV head, fp32, 8-bit pools, the shared-prefix walk, the planned
bench-style step) and the three multi-token forms (per-tile, split,
workgroup-tiled with both of its passes)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import bench_step, build, check_close, scale_for, to_device, to_storage_np
from tests.test_gpu_fp8 import _code_case
from tests.test_gpu_shared_prefix import _groups_case

pytestmark = pytest.mark.gpu

VALU, MFMA = P.PA_VARIANT_VALU, P.PA_VARIANT_MFMA
D128 = scale_for(128)
# negative 1/sqrt(D), zero, and a negative scale sharp enough that a few
# positions carry most of each row's weight
SCALES = {"neg": -D128, "zero": 0.0, "neg_peaked": -0.5}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _f64(t, dtype):
    return O.as_f64(to_storage_np(t), dtype)


def _w(name, seed, hq, hkv, d, bs, dtype):
    return W.Workload(name, seed, 0, hq, hkv, d, bs, dtype, ("fixed", 0), ("factor", 1.3))


LENS = [0, 1, 17, 33, 513, 1025, 2100]

DECODE_SHAPES = [
    # dtype, hq, hkv, d, bs, variant
    ("bf16", 32, 8, 128, 16, MFMA),
    ("bf16", 32, 8, 128, 16, VALU),
    ("bf16", 8, 8, 128, 32, MFMA),
    ("bf16", 64, 8, 128, 16, MFMA),     # the multi-token per-tile kernel at group 8
    ("f32", 4, 4, 64, 16, VALU),
]


@pytest.mark.parametrize("ptok", [0, 64])
@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "-".join(map(str, s)))
@pytest.mark.parametrize("kind", sorted(SCALES))
def test_decode_scales(dev, kind, shape, ptok):
    dtype, hq, hkv, d, bs, variant = shape
    c = build(_w("scale", 501, hq, hkv, d, bs, dtype), dev, lens=LENS, append=False)
    c.scale = SCALES[kind] if d == 128 else SCALES[kind] * float(np.sqrt(128 / d))
    out = c.decode(variant=variant, partition_tokens=ptok)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    got = _f64(out, dtype)
    check_close(got, c.oracle_all(), dtype, f"decode scale {kind} {shape} ptok {ptok}")
    assert np.array_equal(got[0], np.zeros_like(got[0]))


@pytest.mark.parametrize("kind", ["neg", "zero"])
def test_planned_step_scales(dev, kind):
    # the bench's launch: pa_append_tokens, the partition kernel over a work
    # plan, then the merge
    c = build(_w("scale_step", 503, 32, 8, 128, 16, "bf16"), dev,
              lens=[5, 511, 512, 700, 1600, 3000], append=False)
    c.scale = SCALES[kind]
    out = bench_step(c, seed=3)
    check_close(_f64(out, "bf16"), c.oracle_all(), "bf16", f"planned step scale {kind}")


def _mq(dev, c, q_np, qs, mql, split=False, partition_tokens=0):
    out = torch.full((int(qs[-1]), c.hq, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    P.pa_multi_query(to_device(q_np, "bf16", dev), c.k_pool, c.v_pool, c.tables, c.lens,
                     torch.from_numpy(qs).to(dev), c.scale, out, max_seq_len=c.max_len,
                     max_query_len=mql, split=split, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    return _f64(out, "bf16")


# At 4 query heads per KV head the per-tile kernel serves calls whose
# max_query_len stays below 32 tokens (128 rows), also with the context split
# into partitions; longer chunks take the workgroup-tiled kernel.
MQ_MODES = {"per_tile": ([1, 7, 20, 31, 5], False), "split": ([1, 7, 20, 31, 5], True),
            "tiled": ([1, 7, 33, 100, 129], False)}


@pytest.mark.parametrize("mode", sorted(MQ_MODES))
@pytest.mark.parametrize("kind", sorted(SCALES))
def test_multi_query_scales(dev, kind, mode):
    tqs, split = MQ_MODES[mode]
    lens = [1, 40, 300, 1100, 130]
    assert (4 * max(tqs) >= 128) == (mode == "tiled")      # 128 rows per KV head and up
    c = build(_w("scale_mq", 505, 32, 8, 128, 16, "bf16"), dev, lens=lens, append=False)
    c.scale = SCALES[kind]
    rng = np.random.default_rng(506)
    qs = np.concatenate([[0], np.cumsum(tqs)]).astype(np.int32)
    q_np = W.normal_values((int(qs[-1]), 32, 128), rng, "bf16")
    got = _mq(dev, c, q_np, qs, max(tqs), split=split, partition_tokens=64 if split else 0)
    ref = O.multi_query(O.as_f64(q_np, "bf16"), O.as_f64(c.ok_pool, "bf16"),
                        O.as_f64(c.ov_pool, "bf16"), c.otables, c.olens, qs, c.scale)
    check_close(got, ref, "bf16", f"multi-query scale {kind} {mode}")


def test_tiled_exact_pass_negative_scale(dev):
    # a V value beyond the fast pass's range sends the tiles through the
    # exact (two-term bf16 weights) pass, which takes the same sign fold
    lens, tqs = [300, 1100], [40, 64]
    c = build(_w("scale_exact", 507, 32, 8, 128, 16, "bf16"), dev, lens=lens, append=False)
    c.scale = SCALES["neg_peaked"]
    vp = to_storage_np(c.v_pool).copy()
    phys, off = O.positions_to_rows(c.otables[1], lens[1], 16)
    vp[phys[600], 2, off[600], 9] = W.to_bf16_bits(np.array([-40.0], dtype=np.float32))[0]
    c.v_pool.copy_(to_device(vp, "bf16", dev))
    rng = np.random.default_rng(508)
    qs = np.concatenate([[0], np.cumsum(tqs)]).astype(np.int32)
    q_np = W.normal_values((int(qs[-1]), 32, 128), rng, "bf16")
    got = _mq(dev, c, q_np, qs, max(tqs))
    ref = O.multi_query(O.as_f64(q_np, "bf16"), O.as_f64(c.ok_pool, "bf16"), O.as_f64(vp, "bf16"),
                        c.otables, c.olens, qs, c.scale)
    check_close(got, ref, "bf16", "tiled exact pass, negative scale")


@pytest.mark.parametrize("kind", ["neg", "zero"])
def test_e4m3_decode_scales(dev, kind):
    c, kc, vc = _code_case(dev, 32, 8, 16, [0, 1, 17, 513, 2100], seed=509)
    c.scale = SCALES[kind]
    ks, vs = 0.37, 0.11
    out = torch.empty_like(c.q)
    P.pa_decode_e4m3(c.q, torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev), c.tables,
                     c.lens, c.scale, ks, vs, out, max_seq_len=c.max_len)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    ref = O.decode(O.as_f64(c.oq, "bf16"), O.dequantize_e4m3(kc, ks), O.dequantize_e4m3(vc, vs),
                   c.otables, c.olens, c.scale)
    check_close(_f64(out, "bf16"), ref, "bf16", f"e4m3 decode scale {kind}")


@pytest.mark.parametrize("kind", ["neg", "zero"])
def test_shared_prefix_scales(dev, kind):
    c = _groups_case(511, 32, 8, 16, [(4, 5, [1, 7, 40, 300]), (3, 2, [0, 0, 16])])
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    q = to_device(c["q"], "bf16", dev)
    kp, vp = to_device(c["kp"], "bf16", dev), to_device(c["vp"], "bf16", dev)
    out = torch.full_like(q, float("nan"))
    scale = SCALES[kind]
    P.pa_decode_shared_prefix(q, kp, vp, t(c["tab"]), t(c["lens"]), scale, out,
                              group_start=t(c["gs"]), prefix_lens=t(c["prefix"]),
                              max_group_size=c["max_group"], max_prefix_len=c["max_prefix"],
                              max_seq_len=int(c["lens"].max()))
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    ref = O.decode(O.as_f64(c["q"], "bf16"), O.as_f64(c["kp"], "bf16"), O.as_f64(c["vp"], "bf16"),
                   c["tab"], c["lens"], scale)
    check_close(_f64(out, "bf16"), ref, "bf16", f"shared prefix scale {kind}")
