"""GPU parity of the 8-bit (FP8 E4M3) KV pool: the quantized slot write bit
for bit against the oracle's codes (nearest code to the exact quotient, also
right at the rounding boundaries), and decode over pools of every finite code
against the float64 oracle on the dequantized pools."""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import build, check_close, to_device, to_storage_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


@pytest.mark.parametrize("k_scale,v_scale", [(0.005, 0.02), (1.0, 3.0)])
def test_quantized_slot_write_bitwise(dev, k_scale, v_scale):
    """k_scale 0.005 pushes |x| / scale past 448 (saturation) and gives a few
    subnormal codes; the whole pool must match the oracle's codes."""
    rng = np.random.default_rng(401)
    nb, hkv, bs, d, T = 40, 8, 16, 128, 300
    k_new = W.normal_values((T, hkv, d), rng, "bf16")
    v_new = W.normal_values((T, hkv, d), rng, "bf16")
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[::17] = -1                                        # padding rows write nothing
    kc = torch.zeros((nb, hkv, bs, d), dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    P.pa_reshape_and_cache_e4m3(to_device(k_new, "bf16", dev), to_device(v_new, "bf16", dev),
                                torch.from_numpy(slots).to(dev), kc, vc, k_scale, v_scale)
    okc = np.zeros((nb, hkv, bs, d), dtype=np.uint8)
    ovc = np.zeros_like(okc)
    O.reshape_and_cache_e4m3(O.as_f64(k_new, "bf16").astype(np.float32),
                             O.as_f64(v_new, "bf16").astype(np.float32), slots, okc, ovc,
                             k_scale, v_scale)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    got_k, got_v = kc.cpu().numpy(), vc.cpu().numpy()
    assert np.array_equal(got_k, okc) and np.array_equal(got_v, ovc)
    if k_scale < 0.01:
        assert (okc & 0x7F == 0x7E).any()                  # saturation exercised
        assert ((okc & 0x78) == 0).sum() > 0               # subnormal / zero codes exercised


def test_quantized_slot_write_near_rounding_boundaries(dev):
    """Inputs whose quotient x / scale lies within 2^-24 of a midpoint between
    two codes, or on one: the kernel's codes equal the oracle's (nearest code
    to the exact quotient) bit for bit, including the cases where rounding
    x * float32(1 / scale) instead would pick the other code."""
    rng = np.random.default_rng(403)
    mags = [O.e4m3_value(c) for c in range(0x7F)]
    hkv, d, nb, bs = 2, 128, 4, 16
    differ = 0
    for j in range(48):
        # x (bf16) and a midpoint m; the scale float32(x / m) puts x / scale
        # within one float32 rounding of m, and so do x * 2^k for the other
        # midpoints m * 2^k in the normal range
        k = int(rng.integers(8, 0x76))
        m = (mags[k] + mags[k + 1]) / 2
        x0 = float(O.as_f64(W.to_bf16_bits(np.float32([rng.uniform(0.5, 2.0)])), "bf16")[0])
        if j % 4:
            s = float(np.float32(x0 / m))
        else:
            s = 2.0 ** -int(rng.integers(0, 6))      # power-of-two scale:
            x0 = m * s                               # x / s = m exactly, a tie
        row = np.array([x0 * 2.0 ** e for e in range(-6, 6)], dtype=np.float32)
        row = np.concatenate([row, -row])
        vals = np.resize(row, (2, hkv, d)).astype(np.float32)
        bits = W.to_bf16_bits(vals)
        assert np.array_equal(O.as_f64(bits, "bf16"), vals.astype(np.float64))
        slots = np.array([3, 40], dtype=np.int64)
        kc = torch.zeros((nb, hkv, bs, d), dtype=torch.uint8, device=dev)
        vc = torch.zeros_like(kc)
        kb = to_device(bits, "bf16", dev)
        P.pa_reshape_and_cache_e4m3(kb, kb, torch.from_numpy(slots).to(dev), kc, vc, s, s)
        okc = np.zeros((nb, hkv, bs, d), dtype=np.uint8)
        ovc = np.zeros_like(okc)
        O.reshape_and_cache_e4m3(vals, vals, slots, okc, ovc, s, s)
        torch.cuda.synchronize()
        assert np.array_equal(kc.cpu().numpy(), okc), f"case {j}: scale {s!r}, x {x0!r}"
        assert np.array_equal(vc.cpu().numpy(), ovc)
        inv = np.float32(1) / np.float32(s)
        differ += int((O.e4m3_encode((vals * inv).astype(np.float32)) != O.quantize_e4m3(vals, s)).sum())
    assert P.pa_device_errors() == 0
    assert differ > 0            # the reciprocal rule would have failed somewhere


def _code_case(dev, hq, hkv, bs, lens, seed=411):
    """A decode case over code pools holding every finite code of both signs
    (magnitudes 2^-9 .. 448). q is scaled by 1/16 (exact in bf16) so that
    scores over codes up to 448 x k_scale stay a few units wide and the
    softmax mixes several positions."""
    w = W.Workload("f8", seed, 0, hq, hkv, 128, bs, "bf16", ("fixed", 0), ("factor", 1.3))
    c = build(w, dev, lens=lens, append=False)
    rng = np.random.default_rng(seed + 7)
    kc = W.random_e4m3_codes((c.nb, hkv, bs, 128), rng)
    vc = W.random_e4m3_codes((c.nb, hkv, bs, 128), rng)
    c.oq = W.to_bf16_bits((O.as_f64(c.oq, "bf16") / 16).astype(np.float32))
    c.q = to_device(c.oq, "bf16", dev)
    return c, kc, vc


@pytest.mark.parametrize("hq,hkv,bs", [(32, 8, 16), (8, 8, 32), (16, 8, 128), (32, 8, 64)])
@pytest.mark.parametrize("ptok", [0, -1])
def test_decode_over_code_pools(dev, hq, hkv, bs, ptok):
    lens = [0, 1, 15, 16, 17, 33, 511, 512, 513, 1025, 2100]
    c, kc, vc = _code_case(dev, hq, hkv, bs, lens)
    ks, vs = 0.37, 0.11
    out = torch.empty_like(c.q)
    P.pa_decode_e4m3(c.q, torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev), c.tables,
                     c.lens, c.scale, ks, vs, out, max_seq_len=c.max_len, partition_tokens=ptok)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    ref = O.decode(O.as_f64(c.oq, "bf16"), O.dequantize_e4m3(kc, ks), O.dequantize_e4m3(vc, vs),
                   c.otables, c.olens, c.scale)
    got = O.as_f64(to_storage_np(out), "bf16")
    check_close(got, ref, "bf16", f"e4m3 decode {hq}/{hkv} bs {bs} ptok {ptok}")
    assert np.array_equal(got[0], np.zeros_like(got[0]))


def test_shared_kv_hint_same_bits(dev):
    """The shared-blocks hint only changes the loads' cache policy."""
    c, kc, vc = _code_case(dev, 32, 8, 16, [0, 17, 513, 1025, 2100])
    kc_t, vc_t = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    outs = []
    for variant in (P.PA_VARIANT_AUTO, P.PA_DECODE_SHARED_KV):
        out = torch.full_like(c.q, float("nan"))
        P.pa_decode_e4m3(c.q, kc_t, vc_t, c.tables, c.lens, c.scale, 0.37, 0.11, out,
                         max_seq_len=c.max_len, variant=variant)
        outs.append(out)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ref = O.decode(O.as_f64(c.oq, "bf16"), O.dequantize_e4m3(kc, 0.37), O.dequantize_e4m3(vc, 0.11),
                   c.otables, c.olens, c.scale)
    check_close(O.as_f64(to_storage_np(outs[1]), "bf16"), ref, "bf16", "e4m3 hint")


def test_nan_codes_outside_sequences_do_not_leak(dev):
    lens = [5, 16, 17, 600, 1300]
    c, kc, vc = _code_case(dev, 32, 8, 16, lens, seed=421)
    live = np.zeros((c.nb, 16), dtype=bool)
    for i, L in enumerate(lens):
        phys, off = O.positions_to_rows(c.otables[i], L, 16)
        live[phys, off] = True
    kc.transpose(0, 2, 1, 3)[~live] = 0x7F
    vc.transpose(0, 2, 1, 3)[~live] = 0xFF
    out = torch.empty_like(c.q)
    P.pa_decode_e4m3(c.q, torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev), c.tables,
                     c.lens, c.scale, 0.5, 0.5, out, max_seq_len=c.max_len)
    ref = O.decode(O.as_f64(c.oq, "bf16"), O.dequantize_e4m3(kc, 0.5), O.dequantize_e4m3(vc, 0.5),
                   c.otables, c.olens, c.scale)
    got = O.as_f64(to_storage_np(out), "bf16")
    assert np.isfinite(got).all()
    check_close(got, ref, "bf16", "e4m3 nan poison")


@pytest.mark.parametrize("hq,hkv,bs", [(32, 8, 16), (8, 8, 32), (32, 8, 64)])
@pytest.mark.parametrize("ptok", [1024, 256, -1])
def test_planned_decode_over_code_pools(dev, hq, hkv, bs, ptok):
    """pa_decode_e4m3 over a work plan: bitwise equal to the unplanned call at the same
    explicit partition length, within tolerance of the oracle."""
    lens = [0, 1, 15, 16, 17, 33, 511, 512, 513, 1025, 2100, 1024]
    c, kc, vc = _code_case(dev, hq, hkv, bs, lens)
    kc_t, vc_t = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    shape = P._decode_shape(c.q, kc_t, c.tables, c.max_len, ptok, P.PA_VARIANT_MFMA)
    plan = torch.from_numpy(P.pa_decode_plan(shape, c.olens)).to(dev)
    outs = []
    for wp in (None, plan):
        out = torch.full_like(c.q, float("nan"))
        P.pa_decode_e4m3(c.q, kc_t, vc_t, c.tables, c.lens, c.scale, 0.37, 0.11, out,
                         max_seq_len=c.max_len, partition_tokens=ptok, work_plan=wp)
        outs.append(out)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ref = O.decode(O.as_f64(c.oq, "bf16"), O.dequantize_e4m3(kc, 0.37), O.dequantize_e4m3(vc, 0.11),
                   c.otables, c.olens, c.scale)
    check_close(O.as_f64(to_storage_np(outs[1]), "bf16"), ref, "bf16", f"e4m3 planned {ptok}")
    # the automatic length of 8-bit pools is not the plan's: refused on the host
    with pytest.raises(P.PaError):
        P.pa_decode_e4m3(c.q, kc_t, vc_t, c.tables, c.lens, c.scale, 0.37, 0.11, outs[0],
                         max_seq_len=c.max_len, partition_tokens=0, work_plan=plan)


def test_subnormal_codes_reach_the_scores_and_outputs(dev):
    """K and V codes drawn only from the E4M3 subnormals (2^-9 .. 7 * 2^-9)
    and zero, scale 1: with large q the scores depend on them entirely, and the
    outputs are of their size, so a conversion that flushed subnormals would
    fail against the oracle."""
    c, _, _ = _code_case(dev, 32, 8, 16, [1, 17, 300, 513, 1025])
    rng = np.random.default_rng(419)
    shape = (c.nb, c.hkv, 16, 128)
    kc = (rng.integers(0, 8, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)
    vc = (rng.integers(1, 8, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)
    q_np = (W.normal_values(tuple(c.q.shape), rng, "f32") * 1024).astype(np.float32)
    q_bits = W.to_bf16_bits(q_np)
    q = to_device(q_bits, "bf16", dev)
    out = torch.empty_like(q)
    P.pa_decode_e4m3(q, torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev), c.tables,
                     c.lens, c.scale, 1.0, 1.0, out, max_seq_len=c.max_len, partition_tokens=512)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    ref = O.decode(O.as_f64(q_bits, "bf16"), O.dequantize_e4m3(kc, 1.0),
                   O.dequantize_e4m3(vc, 1.0), c.otables, c.olens, c.scale)
    # the test bites: K flushed to zero would give uniform weights (the mean of
    # the V rows), V flushed to zero would give zeros; both are far from ref
    flat = O.decode(O.as_f64(q_bits, "bf16") * 0.0, O.dequantize_e4m3(kc, 1.0),
                    O.dequantize_e4m3(vc, 1.0), c.otables, c.olens, c.scale)
    assert np.abs(flat - ref).max() > 0.01 and np.abs(ref).max() > 0.01
    check_close(O.as_f64(to_storage_np(out), "bf16"), ref, "bf16", "e4m3 subnormal codes")
