"""Pins of the oracle's multi-token query attention (several new tokens per
sequence, causal inside the chunk) against what the mathematics fixes: the
one-token case is the (separately pinned) decode, full-sequence chunks are
torch's causal scaled_dot_product_attention in float64 (a library routine),
partial chunks are the same routine with an explicit mask, plus brute force
and placement invariance."""
import math

import numpy as np
import pytest
import torch

from oracle import pa_oracle as O


def _paged(rng, lens, hkv, d, bs, extra_blocks=5):
    nblk = [O.blocks_needed(L, bs) for L in lens]
    nb = sum(nblk) + extra_blocks
    order = rng.permutation(nb)
    kp = rng.standard_normal((nb, hkv, bs, d))
    vp = rng.standard_normal((nb, hkv, bs, d))
    maxb = max(nblk)
    tab = np.full((len(lens), maxb), -1, dtype=np.int64)
    p = 0
    for i, n in enumerate(nblk):
        tab[i, :n] = order[p:p + n]
        p += n
    return kp, vp, tab


def _contig(pool, table, L, g):
    phys, off = O.positions_to_rows(table, L, pool.shape[2])
    return pool[phys, g, off, :]


def test_one_token_per_sequence_is_decode():
    rng = np.random.default_rng(1)
    lens = [1, 17, 40, 3]
    kp, vp, tab = _paged(rng, lens, 2, 8, 16)
    q = rng.standard_normal((4, 6, 8))
    qs = np.arange(5)
    got = O.multi_query(q, kp, vp, tab, lens, qs, 0.35)
    want = O.decode(q, kp, vp, tab, np.array(lens), 0.35)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_full_prefill_equals_torch_causal_sdpa(hq, hkv):
    rng = np.random.default_rng(2)
    lens = [23, 40]
    d, bs = 16, 8
    kp, vp, tab = _paged(rng, lens, hkv, d, bs)
    q = rng.standard_normal((sum(lens), hq, d))
    qs = np.concatenate([[0], np.cumsum(lens)])
    scale = 1.0 / math.sqrt(d)
    got = O.multi_query(q, kp, vp, tab, lens, qs, scale)
    G = hq // hkv
    for i, L in enumerate(lens):
        for h in range(hq):
            K = torch.from_numpy(_contig(kp, tab[i], L, h // G))
            V = torch.from_numpy(_contig(vp, tab[i], L, h // G))
            Q = torch.from_numpy(q[qs[i]:qs[i + 1], h])
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[None], K[None], V[None], is_causal=True, scale=scale)[0].numpy()
            assert np.allclose(got[qs[i]:qs[i + 1], h], ref, rtol=1e-12, atol=1e-12)


def test_partial_chunk_equals_sdpa_with_offset_causal_mask():
    rng = np.random.default_rng(3)
    lens, tq = [50, 33], [7, 33]
    d, bs, hq, hkv = 8, 16, 4, 2
    kp, vp, tab = _paged(rng, lens, hkv, d, bs)
    qs = np.concatenate([[0], np.cumsum(tq)])
    q = rng.standard_normal((qs[-1], hq, d))
    got = O.multi_query(q, kp, vp, tab, lens, qs, 0.2)
    for i, L in enumerate(lens):
        t = np.arange(tq[i])[:, None]
        p = np.arange(L)[None, :]
        mask = torch.from_numpy(p <= L - tq[i] + t)          # True = attend
        for h in range(hq):
            K = torch.from_numpy(_contig(kp, tab[i], L, h // 2))
            V = torch.from_numpy(_contig(vp, tab[i], L, h // 2))
            Q = torch.from_numpy(q[qs[i]:qs[i + 1], h])
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[None], K[None], V[None], attn_mask=mask[None], scale=0.2)[0].numpy()
            assert np.allclose(got[qs[i]:qs[i + 1], h], ref, rtol=1e-12, atol=1e-12)


def test_brute_force_tiny():
    rng = np.random.default_rng(4)
    lens, tq = [9], [4]
    d, bs = 3, 4
    kp, vp, tab = _paged(rng, lens, 1, d, bs)
    q = rng.standard_normal((4, 2, d))
    got = O.multi_query(q, kp, vp, tab, lens, [0, 4], 0.7)
    for t in range(4):
        for h in range(2):
            npos = 9 - 4 + t + 1
            sc, rows = [], []
            for pos in range(npos):
                b, o = int(tab[0][pos // bs]), pos % bs
                sc.append(0.7 * sum(q[t, h, e] * kp[b, 0, o, e] for e in range(d)))
                rows.append(vp[b, 0, o])
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            ref = [sum(w[k] * rows[k][e] for k in range(npos)) / sum(w) for e in range(d)]
            assert np.allclose(got[t, h], ref, rtol=1e-12, atol=1e-12)


def test_last_chunk_token_sees_everything_first_sees_prefix():
    """Closed forms at the chunk's edges: with V constant per position the
    output is the mean over exactly the attended positions (q = 0)."""
    rng = np.random.default_rng(5)
    L, tq, bs = 20, 5, 8
    kp, vp, tab = _paged(rng, [L], 1, 2, bs)
    for pos in range(L):
        b, o = int(tab[0][pos // bs]), pos % bs
        vp[b, 0, o] = [pos, 1.0]
    q = np.zeros((tq, 1, 2))
    got = O.multi_query(q, kp, vp, tab, [L], [0, tq], 1.0)
    for t in range(tq):
        n = L - tq + t + 1
        assert got[t, 0, 0] == pytest.approx((n - 1) / 2, abs=1e-12)
        assert got[t, 0, 1] == pytest.approx(1.0, abs=1e-15)


def test_placement_invariance_bitwise():
    rng = np.random.default_rng(6)
    lens, tq = [37, 12], [6, 12]
    bs, hkv, d = 8, 2, 4
    kp, vp, tab = _paged(rng, lens, hkv, d, bs, extra_blocks=0)
    nb = kp.shape[0]
    perm = rng.permutation(nb)
    inv = np.argsort(perm)
    kp2, vp2 = kp[inv], vp[inv]            # block b moves to perm[b]
    tab2 = np.where(tab >= 0, perm[np.maximum(tab, 0)], -1)
    qs = [0, 6, 18]
    q = rng.standard_normal((18, 4, d))
    a = O.multi_query(q, kp, vp, tab, lens, qs, 0.5)
    b = O.multi_query(q, kp2, vp2, tab2, lens, qs, 0.5)
    assert np.array_equal(a, b)
