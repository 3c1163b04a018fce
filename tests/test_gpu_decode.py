"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
small and edge-case inputs, compared element by element, plus invariants
that must hold bitwise on the GPU."""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import build, check_close, to_device, to_storage_np

pytestmark = pytest.mark.gpu

VALU, MFMA = P.PA_VARIANT_VALU, P.PA_VARIANT_MFMA


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _f64(t, dtype):
    return O.as_f64(to_storage_np(t), dtype)


def _custom(name, seed, hq, hkv, d, bs, dtype, pool_factor=1.3):
    return W.Workload(name, seed, 0, hq, hkv, d, bs, dtype, ("fixed", 0), ("factor", pool_factor))


EDGE_LENS = [0, 1, 15, 16, 17, 31, 33, 511, 512, 513, 1023, 1025, 1537]

SHAPES = [
    # dtype, hq, hkv, d, bs, variant
    ("bf16", 32, 8, 128, 16, MFMA),
    ("bf16", 32, 8, 128, 16, VALU),
    ("bf16", 8, 8, 128, 16, MFMA),
    ("bf16", 8, 8, 128, 16, VALU),
    ("bf16", 8, 4, 128, 16, MFMA),
    ("bf16", 32, 8, 128, 32, MFMA),
    ("bf16", 32, 8, 128, 8, MFMA),
    ("bf16", 32, 8, 128, 64, MFMA),
    ("bf16", 32, 8, 128, 128, MFMA),
    ("bf16", 8, 8, 128, 8, MFMA),
    ("bf16", 16, 8, 128, 128, MFMA),
    ("bf16", 64, 8, 128, 16, MFMA),     # group 8 and 16: the multi-token per-tile kernel
    ("bf16", 32, 4, 128, 64, MFMA),
    ("bf16", 16, 1, 128, 32, MFMA),
    ("bf16", 32, 2, 128, 128, MFMA),
    ("bf16", 16, 8, 128, 32, VALU),
    ("bf16", 16, 2, 64, 16, VALU),
    ("bf16", 4, 4, 64, 32, VALU),
    ("f32", 4, 4, 64, 16, VALU),
    ("f32", 8, 2, 128, 32, VALU),
    ("f32", 16, 2, 128, 16, VALU),
    ("f32", 2, 1, 64, 32, VALU),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_edge_lengths_all_outputs(dev, shape):
    dtype, hq, hkv, d, bs, variant = shape
    w = _custom("edge", 101, hq, hkv, d, bs, dtype)
    c = build(w, dev, lens=EDGE_LENS, append=False)
    out = c.decode(variant=variant)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    got = _f64(out, dtype)
    ref = c.oracle_all()
    check_close(got, ref, dtype, f"edge {shape}")
    assert np.array_equal(got[0], np.zeros_like(got[0]))


@pytest.mark.parametrize("ptok", [-1, 16, 32, 64, 512, 1024])
@pytest.mark.parametrize("variant", [VALU, MFMA])
def test_partition_lengths(dev, ptok, variant):
    w = _custom("parts", 102, 32, 8, 128, 16, "bf16")
    c = build(w, dev, lens=[1, 100, 511, 700, 2047, 2500])
    ref = c.oracle_all()
    out = c.decode(variant=variant, partition_tokens=ptok)
    check_close(_f64(out, "bf16"), ref, "bf16", f"partition {ptok}")
    assert P.pa_device_errors() == 0


@pytest.mark.parametrize("bs", [8, 64, 128])
@pytest.mark.parametrize("ptok", [-1, 128, 512])
def test_block_sizes_with_partitions(dev, bs, ptok):
    """Block sizes other than 16/32 on the matrix-core kernel, including
    8-token blocks (a 16-token chunk spans two blocks) and blocks longer than
    a partition of 128 tokens' worth of chunks."""
    if ptok > 0 and ptok % bs:
        pytest.skip("partition must be a multiple of the block size")
    w = _custom("bsizes", 104, 32, 8, 128, bs, "bf16")
    c = build(w, dev, lens=[1, 7, 8, 9, 130, 511, 777, 1600])
    out = c.decode(variant=MFMA, partition_tokens=ptok)
    check_close(_f64(out, "bf16"), c.oracle_all(), "bf16", f"bs {bs} ptok {ptok}")
    assert P.pa_device_errors() == 0


def test_single_fp32_workload(dev):
    """33 cached tokens at block size 16 (3 blocks, 15 slack), decode; then
    the 34th token is written to its slot and the step decodes again."""
    w = W.get("single_fp32")
    c = build(w, dev, append=False)
    assert int(c.olens[0]) == 33 and (c.otables[0] >= 0).sum() == 3
    assert O.slack(33, 16) == 15
    out = c.decode()
    check_close(_f64(out, "f32"), c.oracle_all(), "f32", "33 tokens")
    # token 34 -> logical block 2, offset 1
    rng = np.random.default_rng(1234)
    kn = W.normal_values((1, 1, 64), rng, "f32")
    vn = W.normal_values((1, 1, 64), rng, "f32")
    slots, pairs = c.bm.append_slots([0])
    (oslot, ocow), = c.obm.append_slots([0])
    assert slots[0] == oslot == c.otables[0][2] * 16 + 1 and pairs.size == 0 and ocow is None
    P.pa_reshape_and_cache(torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev),
                           torch.from_numpy(slots).to(dev), c.k_pool, c.v_pool)
    O.reshape_and_cache(kn, vn, np.array([oslot]), c.ok_pool, c.ov_pool)
    c.lens.fill_(34)
    c.olens = np.array([34], dtype=np.int32)
    out = c.decode(max_seq_len=34)
    check_close(_f64(out, "f32"), c.oracle_all(), "f32", "34 tokens")
    assert np.array_equal(to_storage_np(c.k_pool), c.ok_pool)
    assert np.array_equal(to_storage_np(c.v_pool), c.ov_pool)


@pytest.mark.parametrize("variant", [VALU, MFMA])
def test_small_mha_workload(dev, variant):
    w = W.get("small_mha")
    c = build(w, dev)
    # the slot write touched exactly the new tokens' rows, bit for bit
    assert np.array_equal(to_storage_np(c.k_pool), c.ok_pool)
    assert np.array_equal(to_storage_np(c.v_pool), c.ov_pool)
    out = c.decode(variant=variant)
    check_close(_f64(out, "bf16"), c.oracle_all(), "bf16", "small_mha")
    assert P.pa_device_errors() == 0


@pytest.mark.parametrize("variant", [VALU, MFMA])
def test_poison_outside_sequences_does_not_change_output(dev, variant):
    w = _custom("poison", 103, 32, 8, 128, 16, "bf16")
    c = build(w, dev, lens=[5, 16, 17, 600, 1300], max_blocks=120)
    base = c.decode(variant=variant).clone()
    used = np.zeros((c.nb, c.bs), bool)
    for i in range(c.B):
        phys, off = O.positions_to_rows(c.otables[i], int(c.olens[i]), c.bs)
        used[phys, off] = True
    mask = torch.from_numpy(~used).to(dev)
    nan = torch.tensor(float("nan"), dtype=c.k_pool.dtype, device=dev)
    c.k_pool[:] = torch.where(mask[:, None, :, None], nan, c.k_pool)
    c.v_pool[:] = torch.where(mask[:, None, :, None], nan, c.v_pool)
    # padding entries past each table's end point at in-range garbage blocks
    tab = c.tables.cpu().numpy()
    rng = np.random.default_rng(5)
    pad = tab < 0
    tab[pad] = rng.integers(0, c.nb, pad.sum())
    c.tables.copy_(torch.from_numpy(tab))
    out = c.decode(variant=variant)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))
    assert P.pa_device_errors() == 0


@pytest.mark.parametrize("variant", [VALU, MFMA])
def test_deterministic_and_placement_invariant(dev, variant):
    w = _custom("perm", 104, 32, 8, 128, 16, "bf16")
    c = build(w, dev, lens=[3, 40, 777, 1500])
    a = c.decode(variant=variant).clone()
    b = c.decode(variant=variant)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # relabel every physical block: pool'[pi(b)] = pool[b], table' = pi(table)
    pi = torch.from_numpy(np.random.default_rng(6).permutation(c.nb)).to(dev)
    kp2, vp2 = torch.empty_like(c.k_pool), torch.empty_like(c.v_pool)
    kp2[pi], vp2[pi] = c.k_pool, c.v_pool
    tab = c.tables.long()
    tab2 = torch.where(tab >= 0, pi[tab.clamp(min=0)], tab).int()
    out = torch.empty_like(c.q)
    P.pa_decode(c.q, kp2, vp2, tab2.contiguous(), c.lens, c.scale, out, max_seq_len=c.max_len,
                variant=variant)
    assert torch.equal(out.view(torch.int16), a.view(torch.int16))


@pytest.mark.parametrize("variant", [VALU, MFMA])
def test_shared_blocks_equal_private_copies(dev, variant):
    w = _custom("share", 105, 32, 8, 128, 16, "bf16")
    c = build(w, dev, lens=[900, 900], append=False, nb=200)
    tab = c.tables.clone()
    # sequence 1 reads sequence 0's blocks (shared) ...
    tab[1] = tab[0]
    q = c.q.clone()
    q[1] = q[0]
    out_shared = torch.empty_like(q)
    P.pa_decode(q, c.k_pool, c.v_pool, tab, c.lens, c.scale, out_shared, max_seq_len=900, variant=variant)
    # ... versus private copies of the same blocks
    n = (tab[0] >= 0).sum().item()
    used = set(tab[0, :n].tolist())
    free = [b for b in range(c.nb) if b not in used][:n]
    for k in range(n):
        c.k_pool[free[k]] = c.k_pool[tab[0, k]]
        c.v_pool[free[k]] = c.v_pool[tab[0, k]]
    tab[1, :n] = torch.tensor(free, dtype=torch.int32, device=dev)
    out_priv = torch.empty_like(q)
    P.pa_decode(q, c.k_pool, c.v_pool, tab, c.lens, c.scale, out_priv, max_seq_len=900, variant=variant)
    assert torch.equal(out_shared.view(torch.int16), out_priv.view(torch.int16))
    assert torch.equal(out_shared[0].view(torch.int16), out_shared[1].view(torch.int16))


def test_split_and_unsplit_agree(dev):
    w = _custom("split", 106, 32, 8, 128, 16, "bf16")
    c = build(w, dev, lens=[4000, 2049, 513])
    ref = c.oracle_all()
    a = _f64(c.decode(partition_tokens=-1), "bf16")
    b = _f64(c.decode(partition_tokens=512), "bf16")
    check_close(a, ref, "bf16", "unsplit")
    check_close(b, ref, "bf16", "split")
    check_close(a, b, "bf16", "split vs unsplit")


def test_variants_agree(dev):
    w = _custom("variants", 107, 32, 8, 128, 16, "bf16")
    c = build(w, dev, lens=list(range(1, 600, 37)))
    a = _f64(c.decode(variant=VALU), "bf16")
    b = _f64(c.decode(variant=MFMA), "bf16")
    check_close(a, b, "bf16", "VALU vs MFMA")


@pytest.mark.parametrize("hq,hkv", [(64, 8), (16, 1)])
@pytest.mark.parametrize("ptok", [-1, 16, 128, 512])
def test_large_groups_partition_lengths(dev, hq, hkv, ptok):
    # group 8 / 16 decode runs on the multi-token per-tile kernel with its
    # context partitions (fp32 partials)
    w = _custom("groups", 110, hq, hkv, 128, 16, "bf16")
    c = build(w, dev, lens=[0, 1, 100, 511, 700, 2047, 2500], append=False)
    out = c.decode(variant=MFMA, partition_tokens=ptok)
    check_close(_f64(out, "bf16"), c.oracle_all(), "bf16", f"group {hq // hkv} ptok {ptok}")
    assert P.pa_device_errors() == 0
    # the automatic choice takes the same path
    auto = c.decode(partition_tokens=ptok)
    assert torch.equal(auto.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (64, 8)])
def test_device_index_errors_are_flagged(dev, hq, hkv):
    w = _custom("errs", 108, hq, hkv, 128, 16, "bf16")
    c = build(w, dev, lens=[40, 70], append=False)
    assert P.pa_device_errors() == 0
    bad = c.tables.clone()
    bad[1, 2] = c.nb + 5                       # out-of-range id at a valid position
    out = torch.empty_like(c.q)
    P.pa_decode(c.q, c.k_pool, c.v_pool, bad, c.lens, c.scale, out, max_seq_len=c.max_len)
    assert P.pa_device_errors() & 0x1
    lens = c.lens.clone()
    lens[0] = c.max_len + 1                    # longer than the host bound
    P.pa_decode(c.q, c.k_pool, c.v_pool, c.tables, lens, c.scale, out, max_seq_len=c.max_len)
    assert P.pa_device_errors() & 0x2
    k = torch.zeros(1, hkv, 128, dtype=torch.bfloat16, device=dev)
    P.pa_reshape_and_cache(k, k, torch.tensor([c.nb * 16], dtype=torch.int64, device=dev),
                           c.k_pool, c.v_pool)
    assert P.pa_device_errors() & 0x4
    P.pa_copy_blocks(c.k_pool, c.v_pool, torch.tensor([[0, c.nb]], dtype=torch.int64, device=dev))
    assert P.pa_device_errors() & 0x8
    assert P.pa_device_errors() == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reshape_and_cache_whole_pool_bitwise(dev, dtype):
    rng = np.random.default_rng(109)
    nb, hkv, bs, d, T = 40, 4, 16, 64, 50
    kp = W.normal_values((nb, hkv, bs, d), rng, dtype)
    vp = W.normal_values((nb, hkv, bs, d), rng, dtype)
    kn = W.normal_values((T, hkv, d), rng, dtype)
    vn = W.normal_values((T, hkv, d), rng, dtype)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[::7] = -1                                   # padding tokens write nothing
    kpt, vpt = to_device(kp, dtype, dev), to_device(vp, dtype, dev)
    P.pa_reshape_and_cache(to_device(kn, dtype, dev), to_device(vn, dtype, dev),
                           torch.from_numpy(slots).to(dev), kpt, vpt)
    O.reshape_and_cache(kn, vn, slots, kp, vp)
    assert np.array_equal(to_storage_np(kpt), kp) and np.array_equal(to_storage_np(vpt), vp)


@pytest.mark.parametrize("block_shape", [(8, 32, 128), (1, 16, 64), (40, 16, 128)])
def test_copy_blocks_whole_pool_bitwise(dev, block_shape):
    hkv, bs, d = block_shape
    rng = np.random.default_rng(110)
    nb = 64
    kp = W.normal_values((nb, hkv, bs, d), rng, "bf16")
    vp = W.normal_values((nb, hkv, bs, d), rng, "bf16")
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:20], perm[20:40]], axis=1).astype(np.int64)
    kpt, vpt = to_device(kp, "bf16", dev), to_device(vp, "bf16", dev)
    P.pa_copy_blocks(kpt, vpt, torch.from_numpy(pairs).to(dev))
    O.copy_blocks(kp, vp, pairs)
    assert np.array_equal(to_storage_np(kpt), kp) and np.array_equal(to_storage_np(vpt), vp)
    assert P.pa_device_errors() == 0
