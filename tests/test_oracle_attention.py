"""Oracle decode attention pinned to things other than itself: a library
routine (torch SDPA in float64 on the CPU), an independent contiguous
formulation, closed forms, invariants and brute force on tiny inputs.

The pin_* helpers take the oracle module so that test_oracle_mutants.py can
run them against deliberately broken copies of it."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import pa_oracle as O


def _scatter_contiguous(k_seq, v_seq, table, nb, bs):
    """Lay contiguous per-sequence K/V [Hkv, L, D] into a pool, one logical
    block slice at a time (tokens contiguous inside each block)."""
    hkv, L, d = k_seq.shape
    kp = np.full((nb, hkv, bs, d), np.nan)
    vp = np.full((nb, hkv, bs, d), np.nan)
    for lb, phys in enumerate(table):
        lo, hi = lb * bs, min(L, (lb + 1) * bs)
        if lo >= hi:
            break
        kp[phys, :, : hi - lo, :] = k_seq[:, lo:hi, :]
        vp[phys, :, : hi - lo, :] = v_seq[:, lo:hi, :]
    return kp, vp


def _case(rng, B, hq, hkv, d, bs, lens, nb=None):
    nblk = [O.blocks_needed(L, bs) for L in lens]
    nb = nb or sum(nblk) + 5
    perm = rng.permutation(nb)
    tables, pos = [], 0
    for n in nblk:
        tables.append([int(x) for x in perm[pos:pos + n]])
        pos += n
    maxb = max(nblk + [1])
    tab = np.full((B, maxb), -1, dtype=np.int64)
    for i, t in enumerate(tables):
        tab[i, :len(t)] = t
    q = rng.standard_normal((B, hq, d))
    kseqs = [rng.standard_normal((hkv, L, d)) for L in lens]
    vseqs = [rng.standard_normal((hkv, L, d)) for L in lens]
    kp = np.full((nb, hkv, bs, d), np.nan)
    vp = np.full((nb, hkv, bs, d), np.nan)
    for i in range(B):
        k1, v1 = _scatter_contiguous(kseqs[i], vseqs[i], tables[i], nb, bs)
        used = np.isfinite(k1)
        kp[used] = k1[used]
        vp[used] = v1[used]
    return q, kp, vp, tab, np.array(lens), kseqs, vseqs


def pin_contiguous_sdpa(O):
    rng = np.random.default_rng(11)
    B, hq, hkv, d, bs = 3, 4, 2, 16, 4
    lens = [1, 9, 23]
    q, kp, vp, tab, sl, ks, vs = _case(rng, B, hq, hkv, d, bs, lens)
    scale = 1.0 / math.sqrt(d)
    got = O.decode(q, kp, vp, tab, sl, scale)
    for i in range(B):
        for h in range(hq):
            g = h // (hq // hkv)
            qq = torch.tensor(q[i, h]).view(1, 1, 1, d)
            kk = torch.tensor(ks[i][g]).view(1, 1, -1, d)
            vv = torch.tensor(vs[i][g]).view(1, 1, -1, d)
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
            np.testing.assert_allclose(got[i, h], ref.view(-1).numpy(), rtol=1e-12, atol=1e-13)


def pin_negative_scale_sdpa(O):
    # any finite scale is accepted; a negative one turns the largest dot
    # product into the smallest weight (library routine: SDPA in float64)
    rng = np.random.default_rng(12)
    B, hq, hkv, d, bs = 2, 4, 1, 8, 4
    lens = [7, 18]
    q, kp, vp, tab, sl, ks, vs = _case(rng, B, hq, hkv, d, bs, lens)
    for scale in (-1.0 / math.sqrt(d), -2.5):
        got = O.decode(q, kp, vp, tab, sl, scale)
        for i in range(B):
            for h in range(hq):
                qq = torch.tensor(q[i, h]).view(1, 1, 1, d)
                kk = torch.tensor(ks[i][0]).view(1, 1, -1, d)
                vv = torch.tensor(vs[i][0]).view(1, 1, -1, d)
                ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
                np.testing.assert_allclose(got[i, h], ref.view(-1).numpy(), rtol=1e-12, atol=1e-13)


def pin_contiguous_dense(O):
    # same layout check with an arbitrary scale and an MHA shape
    rng = np.random.default_rng(12)
    B, hq, hkv, d, bs = 2, 3, 3, 8, 16
    lens = [33, 16]
    q, kp, vp, tab, sl, ks, vs = _case(rng, B, hq, hkv, d, bs, lens)
    got = O.decode(q, kp, vp, tab, sl, 0.37)
    for i in range(B):
        for h in range(hq):
            s = 0.37 * ks[i][h] @ q[i, h]
            e = np.exp(s - s.max())
            np.testing.assert_allclose(got[i, h], e @ vs[i][h] / e.sum(), rtol=1e-12, atol=1e-13)


def pin_gqa_mapping(O):
    # V rows of KV head g all equal g+1: query head h must return h//G + 1
    rng = np.random.default_rng(13)
    B, hq, hkv, d, bs = 2, 8, 2, 4, 4
    lens = [7, 12]
    q, kp, vp, tab, sl, _, _ = _case(rng, B, hq, hkv, d, bs, lens)
    for g in range(hkv):
        vp[:, g] = g + 1.0
    got = O.decode(q, kp, vp, tab, sl, 0.5)
    for h in range(hq):
        np.testing.assert_allclose(got[:, h], h // (hq // hkv) + 1.0, rtol=1e-14)


def pin_closed_forms(O):
    rng = np.random.default_rng(14)
    d, bs = 8, 4
    q, kp, vp, tab, sl, ks, vs = _case(rng, 1, 1, 1, d, bs, [11])
    # q = 0: every weight is equal, the output is the mean of the V rows
    got = O.decode(np.zeros_like(q), kp, vp, tab, sl, 1.0)
    np.testing.assert_allclose(got[0, 0], vs[0][0].mean(axis=0), rtol=1e-13, atol=1e-14)
    # scale = 0: same
    got = O.decode(q, kp, vp, tab, sl, 0.0)
    np.testing.assert_allclose(got[0, 0], vs[0][0].mean(axis=0), rtol=1e-13, atol=1e-14)
    # one score 40 above all others: output is that V row to within e^-40
    qd = np.zeros((1, 1, d)); qd[0, 0, 0] = 1.0
    kp2 = kp.copy(); kp2[..., 0] = 0.0
    t = tab[0]
    kp2[t[5 // bs], 0, 5 % bs, 0] = 40.0
    got = O.decode(qd, kp2, vp, tab, sl, 1.0)
    np.testing.assert_allclose(got[0, 0], vs[0][0][5], atol=1e-15 * 10 + 11 * math.exp(-40) * 10)
    # a single cached token: the output is its V row exactly
    got = O.decode(q, kp, vp, tab, np.array([1]), 3.0)
    assert np.array_equal(got[0, 0], vs[0][0][0])


def pin_bruteforce(O):
    rng = np.random.default_rng(15)
    bs, d, hq, hkv = 4, 3, 2, 1
    for lens in ([1, 5], [8, 13], [40, 2]):
        q, kp, vp, tab, sl, _, _ = _case(rng, 2, hq, hkv, d, bs, lens)
        scale = 0.8
        got = O.decode(q, kp, vp, tab, sl, scale)
        for i in range(2):
            for h in range(hq):
                rows = []
                for p in range(lens[i]):
                    b = int(tab[i][p // bs])
                    rows.append((b, p % bs))
                sc = [scale * sum(float(q[i, h, e]) * float(kp[b, 0, o, e]) for e in range(d)) for b, o in rows]
                mx = max(sc)
                ws = [math.exp(s - mx) for s in sc]
                tot = sum(ws)
                for e in range(d):
                    ref = sum(w * float(vp[b, 0, o, e]) for w, (b, o) in zip(ws, rows)) / tot
                    assert abs(got[i, h, e] - ref) <= 1e-12 * (1 + abs(ref))


ALL_PINS = [pin_contiguous_sdpa, pin_negative_scale_sdpa, pin_contiguous_dense, pin_gqa_mapping, pin_closed_forms, pin_bruteforce]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pins(pin):
    pin(O)


def test_permutation_invariance_bitwise():
    rng = np.random.default_rng(21)
    q, kp, vp, tab, sl, _, _ = _case(rng, 3, 4, 2, 8, 4, [5, 17, 30], nb=40)
    base = O.decode(q, kp, vp, tab, sl, 0.3)
    for _ in range(3):
        pi = rng.permutation(kp.shape[0])
        kp2 = np.empty_like(kp); vp2 = np.empty_like(vp)
        kp2[pi] = kp; vp2[pi] = vp
        tab2 = np.where(tab >= 0, pi[np.maximum(tab, 0)], -1)
        assert np.array_equal(O.decode(q, kp2, vp2, tab2, sl, 0.3), base)


def test_shared_prefix_equals_duplicated_bitwise():
    rng = np.random.default_rng(22)
    bs, d, hkv, hq = 4, 8, 2, 4
    L = 14
    kp = rng.standard_normal((12, hkv, bs, d)); vp = rng.standard_normal((12, hkv, bs, d))
    shared = [3, 7, 1, 9]
    # duplicate every shared block into private copies for sequence 1
    priv = [0, 2, 4, 5]
    kp[priv] = kp[shared]; vp[priv] = vp[shared]
    q = rng.standard_normal((2, hq, d)); q[1] = q[0]
    tab_shared = np.array([shared, shared]); tab_dup = np.array([shared, priv])
    a = O.decode(q, kp, vp, tab_shared, np.array([L, L]), 0.5)
    b = O.decode(q, kp, vp, tab_dup, np.array([L, L]), 0.5)
    assert np.array_equal(a, b) and np.array_equal(a[0], a[1])


def test_poison_outside_the_sequence_is_ignored():
    rng = np.random.default_rng(23)
    q, kp, vp, tab, sl, _, _ = _case(rng, 2, 2, 2, 8, 4, [6, 9], nb=12)
    assert np.isnan(kp).any()          # slack and unused blocks hold NaN
    out = O.decode(q, kp, vp, tab, sl, 0.4)
    assert np.isfinite(out).all()


def test_zero_length_gives_zeros():
    rng = np.random.default_rng(24)
    q, kp, vp, tab, sl, _, _ = _case(rng, 2, 2, 1, 4, 4, [0, 3])
    out = O.decode(q, kp, vp, tab, sl, 1.0)
    assert np.array_equal(out[0], np.zeros((2, 4))) and np.isfinite(out[1]).all()


@pytest.mark.parametrize("ptok", [4, 8, 12, 64])
def test_partitioned_equals_unsplit(ptok):
    rng = np.random.default_rng(25)
    q, kp, vp, tab, sl, _, _ = _case(rng, 3, 4, 2, 8, 4, [1, 29, 64])
    a = O.decode(q, kp, vp, tab, sl, 0.6)
    b = O.decode_partitioned(q, kp, vp, tab, sl, 0.6, ptok)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-13)


def test_bf16_exact_conversion():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -0.0]
    got = O.as_f64(bits, "bf16")
    assert list(got) == want
    x = np.array([1.5, -3.25e-5], dtype=np.float32)
    assert list(O.as_f64(x, "f32")) == [1.5, float(np.float32(-3.25e-5))]


def test_bf16_rounding_of_inputs_is_rne():
    # the shared input generator rounds fp32 draws to bf16 by nearest-even
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    got = O.as_f64(W.to_bf16_bits(x), "bf16")
    assert list(got) == [1.0, 1.0 + 2 * 2.0 ** -7, 1.0 + 2.0 ** -7]


def test_reshape_and_cache_writes_exact_rows_only():
    rng = np.random.default_rng(26)
    nb, hkv, bs, d = 6, 2, 4, 8
    kp = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vp = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    k0, v0 = kp.copy(), vp.copy()
    kn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = np.array([5 * bs + 3, -1, 0])
    O.reshape_and_cache(kn, vn, slots, kp, vp)
    assert np.array_equal(kp[5, :, 3], kn[0]) and np.array_equal(vp[0, :, 0], vn[2])
    changed = np.argwhere((kp != k0).any(axis=-1))
    assert {tuple(x) for x in changed.tolist()} <= {(5, 0, 3), (5, 1, 3), (0, 0, 0), (0, 1, 0)}
    mask = np.ones(kp.shape[:3], bool); mask[5, :, 3] = False; mask[0, :, 0] = False
    assert np.array_equal(kp[mask], k0[mask]) and np.array_equal(vp[mask], v0[mask])


def test_copy_blocks_bitwise():
    rng = np.random.default_rng(27)
    kp = rng.integers(0, 65535, (8, 2, 4, 8)).astype(np.uint16)
    vp = rng.integers(0, 65535, (8, 2, 4, 8)).astype(np.uint16)
    k0, v0 = kp.copy(), vp.copy()
    O.copy_blocks(kp, vp, np.array([[1, 6], [3, 2]]))
    assert np.array_equal(kp[6], k0[1]) and np.array_equal(vp[2], v0[3])
    for b in (0, 1, 3, 4, 5, 7):
        assert np.array_equal(kp[b], k0[b]) and np.array_equal(vp[b], v0[b])
