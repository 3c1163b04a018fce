"""GPU parity of pa_append_tokens: a decode loop whose block tables and
lengths live on the device and follow the host block manager's appends.
After every step the device tables and lengths must equal the oracle block
manager's export bit for bit (new blocks and copy-on-write replacements
included), the pools must equal the oracle's slot writes, and a decode over
the device tables must match the float64 oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_343_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests.paged_case import check_close, scale_for, to_device, to_storage_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f32", 32), ("e4m3", 16)])
def test_append_loop_tracks_host_manager(dev, dtype, bs):
    rng = np.random.default_rng(515)
    hq, hkv, d = 8, 2, 128
    lens0 = [0, 1, 15, 16, 17, 31, 40, 100]
    steps = 40
    B = len(lens0) + 2                 # two forked children of sequence 6 (40 tokens)
    nb = 200
    order = W.free_order(nb, rng)
    bm, ob = P.BlockManager(nb, bs, order), O.OracleBlockManager(nb, bs, order)
    for i, L in enumerate(lens0):
        bm.add_seq(i, L)
        ob.add_seq(i, L)
    for child in (8, 9):               # share every block of sequence 6, partial last one included
        bm.fork(6, child)
        ob.fork(6, child)
    maxb = (max(lens0) + steps) // bs + 2
    ids = list(range(B))
    tab, ln = bm.export(ids, maxb)
    otab, oln = ob.export(ids, maxb)
    assert np.array_equal(tab, otab) and np.array_equal(ln, oln)
    tables = torch.from_numpy(tab).to(dev)
    lens = torch.from_numpy(ln).to(dev)
    fp8 = dtype == "e4m3"
    sdt = "bf16" if fp8 else dtype
    scales = (0.05, 0.07)
    if fp8:
        okp = W.random_e4m3_codes((nb, hkv, bs, d), rng)
        ovp = W.random_e4m3_codes((nb, hkv, bs, d), rng)
        kp, vp = torch.from_numpy(okp.copy()).to(dev), torch.from_numpy(ovp.copy()).to(dev)
    else:
        okp = W.normal_values((nb, hkv, bs, d), rng, dtype)
        ovp = W.normal_values((nb, hkv, bs, d), rng, dtype)
        kp, vp = to_device(okp, dtype, dev), to_device(ovp, dtype, dev)
    cow_total = 0
    P.pa_device_errors()
    for s in range(steps):
        # sequence 3 sits out every third step (a padding slot of -1)
        active = [i for i in ids if not (i == 3 and s % 3 == 0)]
        slots, pairs = bm.append_slots(active)
        ores = ob.append_slots(active)
        assert slots.tolist() == [x for x, _ in ores]
        opairs = [c for _, c in ores if c is not None]
        assert [tuple(p) for p in pairs.tolist()] == opairs
        if len(opairs):
            cow_total += len(opairs)
            P.pa_copy_blocks(kp, vp, torch.from_numpy(pairs).to(dev))
            O.copy_blocks(okp, ovp, np.array(opairs))
        full = np.full(B, -1, dtype=np.int64)
        full[active] = slots
        kn = W.normal_values((B, hkv, d), rng, sdt)
        vn = W.normal_values((B, hkv, d), rng, sdt)
        P.pa_append_tokens(to_device(kn, sdt, dev), to_device(vn, sdt, dev),
                           torch.from_numpy(full).to(dev), kp, vp, tables, lens,
                           kv_scales=scales if fp8 else None)
        if fp8:
            O.reshape_and_cache_e4m3(O.as_f64(kn[active], "bf16").astype(np.float32),
                                     O.as_f64(vn[active], "bf16").astype(np.float32), slots,
                                     okp, ovp, *scales)
        else:
            O.reshape_and_cache(kn[active], vn[active], slots, okp, ovp)
        otab, oln = ob.export(ids, maxb)
        torch.cuda.synchronize()
        assert P.pa_device_errors() == 0
        assert np.array_equal(tables.cpu().numpy(), otab), f"tables differ after step {s}"
        assert np.array_equal(lens.cpu().numpy(), oln), f"lengths differ after step {s}"
    assert cow_total == 2                     # the two children copy the shared partial block
    assert np.array_equal(to_storage_np(kp), okp) and np.array_equal(to_storage_np(vp), ovp)
    # decode over the device-maintained tables
    qn = W.normal_values((B, hq, d), rng, sdt)
    q = to_device(qn, sdt, dev)
    out = torch.empty_like(q)
    sc = scale_for(d)
    ml = int(oln.max())
    if fp8:
        P.pa_decode_e4m3(q, kp, vp, tables, lens, sc, *scales, out, max_seq_len=ml,
                         partition_tokens=64)
        ref = O.decode(O.as_f64(qn, "bf16"), O.dequantize_e4m3(okp, scales[0]),
                       O.dequantize_e4m3(ovp, scales[1]), otab, oln, sc)
    else:
        P.pa_decode(q, kp, vp, tables, lens, sc, out, max_seq_len=ml, partition_tokens=64)
        ref = O.decode(O.as_f64(qn, dtype), O.as_f64(okp, dtype), O.as_f64(ovp, dtype), otab,
                       oln, sc)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == 0
    check_close(O.as_f64(to_storage_np(out), sdt), ref, sdt, f"decode after appends {dtype}")


def test_append_rejects_slot_that_does_not_fit_position(dev):
    bs, hkv, d, nb = 16, 1, 64, 8
    kp = torch.zeros((nb, hkv, bs, d), dtype=torch.float32, device=dev)
    vp = torch.zeros_like(kp)
    tables = torch.tensor([[5, -1], [2, -1], [3, -1]], dtype=torch.int32, device=dev)
    lens = torch.tensor([3, 16, 31], dtype=torch.int32, device=dev)
    k = torch.ones((3, hkv, d), dtype=torch.float32, device=dev)
    # seq 0: position 3 but offset 4; seq 1: position 16 at offset 0 of block 7 (fits);
    # seq 2: position 31 -> entry 1 of 2, but offset 0 is not 31 % 16
    slots = torch.tensor([5 * bs + 4, 7 * bs + 0, 6 * bs + 0], dtype=torch.int64, device=dev)
    P.pa_device_errors()
    P.pa_append_tokens(k, k, slots, kp, vp, tables, lens)
    torch.cuda.synchronize()
    assert P.pa_device_errors() == P.PA_DEVERR_SLOT
    assert tables.cpu().tolist() == [[5, -1], [2, 7], [3, -1]]
    assert lens.cpu().tolist() == [3, 17, 31]
    # the rows themselves are still written to their slots
    assert kp[5, 0, 4].eq(1).all() and kp[7, 0, 0].eq(1).all() and kp[6, 0, 0].eq(1).all()
    # a position past the table
    lens2 = torch.tensor([32, 0, 0], dtype=torch.int32, device=dev)
    P.pa_append_tokens(k[:1], k[:1], slots[:1].clone().fill_(0), kp, vp, tables[:1], lens2[:1])
    torch.cuda.synchronize()
    assert P.pa_device_errors() == P.PA_DEVERR_SLOT
    assert lens2[0].item() == 32
