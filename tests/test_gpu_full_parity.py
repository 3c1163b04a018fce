"""Element-complete GPU parity at the workloads' full sizes, in the launch the
bench times, against the plain-C float64 oracle over every (sequence, head)
row.

Each case builds the workload on both sides from the same draws, then runs
one decode step the way bench.py does: the host block manager reserves the
slots (its oracle mirror must agree), the host builds the work plan from its
lengths, pa_append_tokens writes the new rows and advances the device-resident
tables and lengths (which must equal the mirror's export afterwards), and
pa_decode_partition over the plan + pa_decode_reduce decode
(pa_decode_shared_prefix, its walks over a plan, for the shared-prefix
batches). Every output element is then compared with the
oracle under |got - ref| <= 2e-3 + 1e-2 |ref|, and max-abs / max-rel are
printed per case.

The math is ordinary attention over the gathered rows ("Walk through paged
attention end to end ...", single-decode-step pseudo-code and "Red flags").
Scaling q by 16 or 32 makes the softmax peaked (one or a few positions carry
nearly all the weight), where a partition's partial output is the size of a
single V row; the cancelling-partials case below builds partials of opposite
sign on purpose.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import (TOL, bench_step, build, build_shared_prefix, check_close,
                              to_device, to_storage_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _full_check(c, out, what):
    ref = c.oracle_c()
    got = O.as_f64(to_storage_np(out), c.dtype)
    assert np.isfinite(got).all(), what
    ma, mr = check_close(got, ref, c.dtype, what)
    print(f"{what}: all {got.size} outputs within tolerance; max_abs={ma:.3g} "
          f"max_rel={mr:.3g}", flush=True)
    return got, ref


@pytest.mark.parametrize("name,q_scale", [("llama3_8b", 1), ("llama3_8b", 16),
                                          ("llama2_13b", 1), ("llama2_13b", 32)])
def test_bench_launch_every_row(dev, name, q_scale):
    w = W.get(name)
    ctx = W.draw_lengths(w, np.random.default_rng(w.seed))
    maxb = O.blocks_needed(int(ctx.max()) + 1, w.block_size)
    print(f"full parity {name} q x{q_scale}: building", flush=True)
    c = build(w, dev, pool_on_device=True, append=False, max_blocks=maxb)
    out = bench_step(c, seed=w.seed, q_scale=q_scale)
    _full_check(c, out, f"{name} q x{q_scale}")


@pytest.mark.parametrize("name", ["shared_prefix", "shared_prefix_long"])
def test_shared_prefix_bench_launch_every_row(dev, name):
    """The shared-prefix batch (64 groups x 4 samples of a 1040-token prompt,
    copy-on-write of the half-filled prompt block at setup), alone and with
    16 unshared 32,768-token sequences, through pa_decode_shared_prefix with
    its walks over a plan, as the bench runs it."""
    w = W.get(name)
    print(f"full parity {name}: building", flush=True)
    c = build_shared_prefix(w, dev, final_append=False)
    assert c.extra["cow_pairs"].shape == (64 * 3, 2)
    out = bench_step(c, seed=w.seed, shared_prefix=True)
    _full_check(c, out, name)


def test_cancelling_peaked_partials(dev):
    """Two 512-position partitions per sequence, each dominated by three
    positions of equal score, whose V rows nearly cancel across the two
    partitions: the output is close to zero while each partition's partial
    output is of the size of a V row. fp32 partials (the default) meet the
    tolerance on every element. With PA_DECODE_HALF_PARTIALS the error
    reaches the documented bound 2^-8 * sum_j w_j |o_j| and leaves the
    tolerance, which is why bf16 partials are an option and not the
    default."""
    hq, hkv, d, bs, L, B = 32, 8, 128, 16, 1024, 16
    w = W.Workload("cancel", 97, 0, hq, hkv, d, bs, "bf16", ("fixed", 0), ("factor", 1.0))
    c = build(w, dev, lens=[L] * B, append=False)
    rng = np.random.default_rng(98)
    q = np.zeros((B, hq, d), dtype=np.float32)
    q[:, :, 0] = 32.0
    kp = O.as_f64(c.ok_pool, "bf16").astype(np.float32)
    vp = O.as_f64(c.ov_pool, "bf16").astype(np.float32)
    for i in range(B):
        phys, off = O.positions_to_rows(c.otables[i], L, bs)
        kp[phys, :, off, :] = 0.0
        kp[phys, :, off, 0] = -4.0
        hot = np.concatenate([rng.choice(512, 3, replace=False),
                              512 + rng.choice(512, 3, replace=False)])
        r = rng.standard_normal((3, hkv, d)).astype(np.float32) * 2
        delta = rng.standard_normal((3, hkv, d)).astype(np.float32) * 0.01
        for k, p in enumerate(hot):
            kp[phys[p], :, off[p], 0] = 4.0
            vp[phys[p], :, off[p], :] = r[k % 3] if k < 3 else -r[k % 3] + delta[k % 3]
    c.oq, c.ok_pool, c.ov_pool = W.to_bf16_bits(q), W.to_bf16_bits(kp), W.to_bf16_bits(vp)
    c.q = to_device(c.oq, "bf16", dev)
    c.k_pool.copy_(to_device(c.ok_pool, "bf16", dev))
    c.v_pool.copy_(to_device(c.ov_pool, "bf16", dev))
    ref = c.oracle_c()
    # the documented bound of bf16 partials, from the oracle's own partitions
    q64, k64, v64 = (O.as_f64(x, "bf16") for x in (c.oq, c.ok_pool, c.ov_pool))
    bound = np.zeros_like(ref)
    for i in range(B):
        for h in range(hq):
            parts = O.partition_partials(q64[i, h], k64, v64, c.otables[i], L, c.scale,
                                         O.kv_head_of(h, hq, hkv), bs, 512)
            big = max(p[0] for p in parts)
            wts = np.array([p[1] * np.exp(p[0] - big) for p in parts])
            wts /= wts.sum()
            bound[i, h] = 2.0 ** -8 * sum(wj * np.abs(p[2]) for wj, p in zip(wts, parts))
    assert np.abs(ref).max() < 0.1 < bound.max() * 2 ** 8       # partials ~ V rows, output ~ 0
    outs = {}
    for flag in (0, P.PA_DECODE_HALF_PARTIALS):
        out = torch.full_like(c.q, float("nan"))
        P.pa_decode(c.q, c.k_pool, c.v_pool, c.tables, c.lens, c.scale, out, max_seq_len=L,
                    partition_tokens=512, variant=P.PA_VARIANT_MFMA | flag)
        outs[flag] = out
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    got = O.as_f64(to_storage_np(outs[0]), "bf16")
    ma, mr = check_close(got, ref, "bf16", "cancelling partials, fp32 partials")
    print(f"cancelling partials: fp32 partials max_abs={ma:.3g}", flush=True)
    half = O.as_f64(to_storage_np(outs[P.PA_DECODE_HALF_PARTIALS]), "bf16")
    err = np.abs(half - ref)
    # bf16 partials: inside their bound (plus the output's own rounding)...
    assert (err <= bound * 1.01 + 2.0 ** -8 * np.abs(ref) + 1e-5).all()
    # ...which here is well outside the bf16 tolerance
    atol, rtol = TOL["bf16"]
    print(f"cancelling partials: bf16 partials max_abs={err.max():.3g}, "
          f"{int((err > atol + rtol * np.abs(ref)).sum())} of {err.size} outside tolerance",
          flush=True)
    assert (err > atol + rtol * np.abs(ref)).any()
