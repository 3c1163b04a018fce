"""The plain-C float64 oracle agrees with the numpy oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import pa_oracle as O
from oracle import ref as R


def _build(rng, B, hq, hkv, d, bs, lens, dtype):
    nb = sum(O.blocks_needed(L, bs) for L in lens) + 7
    bm = O.OracleBlockManager(nb, bs, W.free_order(nb, rng))
    for i, L in enumerate(lens):
        bm.add_seq(i, int(L))
    maxb = max(O.blocks_needed(L, bs) for L in lens) + 2
    tab, sl = bm.export(list(range(B)), maxb)
    q = W.normal_values((B, hq, d), rng, dtype)
    kp = W.normal_values((nb, hkv, bs, d), rng, dtype)
    vp = W.normal_values((nb, hkv, bs, d), rng, dtype)
    return q, kp, vp, tab, sl


@pytest.mark.parametrize("dtype,hq,hkv,d,bs", [("f32", 1, 1, 64, 16), ("bf16", 8, 2, 32, 16),
                                               ("bf16", 4, 4, 16, 32), ("f32", 6, 3, 8, 8)])
def test_c_oracle_matches_numpy(dtype, hq, hkv, d, bs):
    rng = np.random.default_rng(31)
    lens = [0, 1, 33, 70, 5]
    q, kp, vp, tab, sl = _build(rng, len(lens), hq, hkv, d, bs, lens, dtype)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    a = O.decode(O.as_f64(q, dtype), O.as_f64(kp, dtype), O.as_f64(vp, dtype), tab, sl, scale)
    b = R.decode(q, kp, vp, tab, sl, scale, dtype, num_threads=2)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)
    assert np.array_equal(b[0], np.zeros_like(b[0]))


def test_c_oracle_rejects_bad_block_id():
    rng = np.random.default_rng(32)
    q, kp, vp, tab, sl = _build(rng, 1, 1, 1, 8, 4, [6], "f32")
    tab[0, 1] = kp.shape[0] + 3
    with pytest.raises(RuntimeError):
        R.decode(q, kp, vp, tab, sl, 1.0, "f32")


@pytest.mark.parametrize("hq,hkv,bs", [(8, 2, 16), (4, 4, 32)])
def test_c_oracle_e4m3_matches_numpy(hq, hkv, bs):
    """8-bit pools over every finite code of both signs: the C oracle reads
    code value times its pool's scale, as the numpy oracle's dequantized
    pools do."""
    rng = np.random.default_rng(33)
    lens = [0, 1, 33, 70, 5]
    q, kp, _, tab, sl = _build(rng, len(lens), hq, hkv, 32, bs, lens, "bf16")
    kc = W.random_e4m3_codes(kp.shape, rng)
    vc = W.random_e4m3_codes(kp.shape, rng)
    q = W.to_bf16_bits(O.as_f64(q, "bf16").astype(np.float32) / 64)
    scale, ks, vs = 0.125, 0.37, 0.11
    a = O.decode(O.as_f64(q, "bf16"), O.dequantize_e4m3(kc, ks), O.dequantize_e4m3(vc, vs),
                 tab, sl, scale)
    b = R.decode_e4m3(q, kc, vc, ks, vs, tab, sl, scale, num_threads=2)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
    assert np.abs(a).max() > 1.0
