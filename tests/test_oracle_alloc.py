"""Oracle block manager mirror: append rule, slots, fork, copy-on-write, free."""
import numpy as np
import pytest

from oracle import pa_oracle as O


def _invariants(bm):
    # each block's count equals the number of tables holding it; free blocks
    # have count 0 and are exactly the blocks no table holds
    held = {}
    for t in bm.tables.values():
        for b in t:
            held[b] = held.get(b, 0) + 1
    for b in range(bm.num_blocks):
        assert bm.ref[b] == held.get(b, 0)
    assert set(bm.free) == {b for b in range(bm.num_blocks) if b not in held}
    assert len(bm.free) + len(held) == bm.num_blocks
    for s, t in bm.tables.items():
        assert len(t) == O.blocks_needed(bm.ntok[s], bm.block_size)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_append_allocates_exactly_on_block_boundary(bs):
    rng = np.random.default_rng(0)
    nb = 64
    bm = O.OracleBlockManager(nb, bs, rng.permutation(nb))
    bm.add_seq(0, 0)
    order = list(bm.free)
    for p in range(5 * bs + 3):
        before = bm.num_free()
        slot, cow = bm.append_slot(0)
        assert cow is None
        # a block is taken iff the position starts a block
        assert before - bm.num_free() == (1 if p % bs == 0 else 0)
        t = bm.table(0)
        assert len(t) == O.blocks_needed(p + 1, bs)
        assert slot == O.slot_of(t, p, bs)
        assert t == order[:len(t)]        # blocks come from the front of the free list
    _invariants(bm)


def test_single_fp32_workload_token_34():
    # 33 cached tokens at block size 16 occupy 3 blocks; the 34th token
    # (position 33) goes to logical block 2 at offset 1 without a new block
    rng = np.random.default_rng(1)
    bm = O.OracleBlockManager(16, 16, rng.permutation(16))
    bm.add_seq(0, 33)
    t = bm.table(0)
    assert len(t) == 3 and bm.num_free() == 13
    slot, cow = bm.append_slot(0)
    assert cow is None and slot == t[2] * 16 + 1 and bm.num_free() == 13
    slot, cow = bm.append_slot(0)
    assert slot == t[2] * 16 + 2


def test_fork_shares_and_cow_copies_partial_block():
    bs = 16
    bm = O.OracleBlockManager(32, bs)
    bm.add_seq(0, 40)                  # blocks 0,1,2 ; last one holds 8 tokens
    for c in (1, 2, 3):
        bm.fork(0, c)
    assert [bm.refcount(b) for b in bm.table(0)] == [4, 4, 4]
    _invariants(bm)
    # writers served in order: the first three copy, the last keeps the original
    pairs = []
    for s in (0, 1, 2, 3):
        slot, cow = bm.append_slot(s)
        pairs.append(cow)
        assert slot == bm.table(s)[2] * bs + 8
    assert pairs[3] is None
    assert [p[0] for p in pairs[:3]] == [2, 2, 2]
    dsts = [p[1] for p in pairs[:3]]
    assert len(set(dsts)) == 3 and 2 not in dsts
    assert bm.table(3)[2] == 2 and bm.refcount(2) == 1
    # full shared blocks stay shared
    assert bm.refcount(0) == 4 and bm.refcount(1) == 4
    for s in range(4):
        assert bm.table(s)[:2] == [0, 1]
    _invariants(bm)


def test_fork_at_block_boundary_needs_no_copy():
    # divergence at a multiple of the block size: the child's next token
    # opens a fresh block and nothing is copied
    bm = O.OracleBlockManager(16, 16)
    bm.add_seq(0, 32)
    bm.fork(0, 1)
    slot, cow = bm.append_slot(1)
    assert cow is None and bm.table(1)[:2] == bm.table(0)
    assert len(bm.table(1)) == 3
    _invariants(bm)


def test_free_returns_blocks_and_respects_sharing():
    bm = O.OracleBlockManager(8, 4, [7, 6, 5, 4, 3, 2, 1, 0])
    bm.add_seq(0, 9)          # 7, 6, 5
    bm.fork(0, 1)
    bm.free_seq(0)
    assert bm.num_free() == 5     # shared blocks stay with sequence 1
    bm.free_seq(1)
    assert list(bm.free) == [4, 3, 2, 1, 0, 7, 6, 5]
    _invariants(bm)


def test_exhaustion_leaves_state_unchanged():
    bm = O.OracleBlockManager(4, 4)
    bm.add_seq(0, 4)
    bm.add_seq(1, 8)
    with pytest.raises(O.OracleNoBlocks):
        bm.add_seq(2, 5)
    snap = (list(bm.free), dict((k, list(v)) for k, v in bm.tables.items()), dict(bm.ntok))
    bm.add_seq(3, 0)
    # both sequences are block-aligned: a batch append needs 2 blocks, 1 free
    with pytest.raises(O.OracleNoBlocks):
        bm.append_slots([0, 1])
    assert list(bm.free) == snap[0] and bm.ntok[0] == 4 and bm.ntok[1] == 8
    _invariants(bm)


def test_random_churn_invariants():
    rng = np.random.default_rng(7)
    bs, nb = 16, 256
    bm = O.OracleBlockManager(nb, bs, rng.permutation(nb))
    live, nxt = [], 0
    for step in range(3000):
        r = rng.random()
        try:
            if r < 0.1 or not live:
                bm.add_seq(nxt, int(rng.integers(0, 80)))
                live.append(nxt); nxt += 1
            elif r < 0.15:
                bm.fork(live[int(rng.integers(len(live)))], nxt)
                live.append(nxt); nxt += 1
            elif r < 0.22:
                s = live.pop(int(rng.integers(len(live))))
                bm.free_seq(s)
            else:
                s = live[int(rng.integers(len(live)))]
                p = bm.ntok[s]
                slot, cow = bm.append_slot(s)
                assert slot == O.slot_of(bm.table(s), p, bs)
                if cow is not None:
                    assert bm.refcount(cow[0]) >= 1 and bm.refcount(cow[1]) == 1
        except O.OracleNoBlocks:
            s = live.pop(0)
            bm.free_seq(s)
        _invariants(bm) if step % 100 == 0 else None
    _invariants(bm)


# -- swapping ([N4N] "Why it matters for KV cache": blocks evicted to CPU
# memory and fetched back when the request resumes) --------------------------

def _check_swap_invariants(ob, ncpu):
    held = {}
    for s, t in ob.tables.items():
        if s in ob.swapped:
            continue
        for b in t:
            held[b] = held.get(b, 0) + 1
    assert all(ob.ref[b] == held.get(b, 0) for b in range(ob.num_blocks))
    assert sorted(list(ob.free) + list(held)) == list(range(ob.num_blocks))
    on_host = [c for s in ob.swapped for c in ob.tables[s]]
    assert sorted(list(ob.swap_free) + on_host) == list(range(ncpu))


def test_oracle_swap_invariants_random_ops():
    rng = np.random.default_rng(31)
    ob = O.OracleBlockManager(300, 16, rng.permutation(300))
    ncpu = 150
    ob.set_swap_space(ncpu)
    for i in range(8):
        ob.add_seq(i, int(rng.integers(1, 150)))
    ob.fork(1, 8); ob.fork(1, 9)
    live = list(range(10))
    for _ in range(200):
        s = int(rng.choice(live))
        op = rng.integers(0, 3)
        try:
            if op == 0:
                ob.swap_out(s)
            elif op == 1:
                ob.swap_in(s)
            elif s not in ob.swapped:
                ob.append_slots([s])
        except (ValueError, O.OracleNoBlocks):
            pass
        _check_swap_invariants(ob, ncpu)


def test_oracle_swap_round_trip_keeps_attention_bitwise():
    """A sequence swapped out, its device blocks reused (poisoned), then
    swapped back into different blocks decodes to the same bits."""
    rng = np.random.default_rng(32)
    bs, nb, hkv, d = 16, 40, 2, 8
    ob = O.OracleBlockManager(nb, bs, rng.permutation(nb))
    ob.set_swap_space(12)
    ob.add_seq(0, 90); ob.add_seq(1, 30)
    kp = rng.standard_normal((nb, hkv, bs, d)); vp = rng.standard_normal((nb, hkv, bs, d))
    hk = np.zeros((12, hkv, bs, d)); hv = np.zeros((12, hkv, bs, d))
    q = rng.standard_normal((2, 4, d))
    tab, lens = ob.export([0, 1], 8)
    before = O.decode(q, kp, vp, tab, lens, 0.3)
    old_blocks = list(tab[0][tab[0] >= 0])
    O.swap_blocks(kp, vp, hk, hv, ob.swap_out(0))
    kp[old_blocks] = np.nan; vp[old_blocks] = np.nan      # freed blocks reused
    ob.add_seq(2, 40)                                      # takes some of them
    moves = ob.swap_in(0)
    O.swap_blocks(hk, hv, kp, vp, moves)
    tab2, lens2 = ob.export([0, 1], 8)
    after = O.decode(q, kp, vp, tab2, lens2, 0.3)
    assert not np.array_equal(tab2[0], tab[0])             # new physical blocks
    assert np.array_equal(before, after)
