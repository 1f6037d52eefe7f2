"""Pins of the oracle's block-pool model (policy and invariants)."""
import random

import pytest
from hypothesis import given, settings, strategies as st

from oracle import layout
from oracle.pool_model import BadSeq, InvalidArg, NoBlocks, PoolModel


def test_printed_block_table(golden):
    """Logical blocks 0,1,2 placed at physical 8,3,11: every token lands there."""
    ex = golden("block_table_example.json")
    phys = ex["physical_blocks"]
    for page in (2, 16):
        pool = PoolModel(16, page)
        sid = pool.seq_create()
        pool.set_table(sid, phys, 3 * page)
        for t in range(3 * page):
            s = pool.slot(sid, t)
            assert s // page == phys[t // page]
            assert s % page == t % page
        assert 8 not in pool.free and 3 not in pool.free and 11 not in pool.free
        pool.check_invariants()


def test_table_grows_by_one_block_per_page():
    pool = PoolModel(8, 4, free_order=[5, 2, 7, 0, 1, 3, 4, 6])
    sid = pool.seq_create()
    seen = []
    for t in range(10):
        pool.append_slots([sid], [1])
        seen.append(len(pool.tables[sid]))
    assert seen == [1, 1, 1, 1, 2, 2, 2, 2, 3, 3]
    assert pool.tables[sid] == [5, 2, 7]          # head of the free list, in order


def test_copy_on_write_three_sharers():
    """Prefix of 3 tokens, page 2: the shared last block is half full.

    The first two sharers to write get private copies; the last one left
    writes in place, so exactly two copies happen.
    """
    pool = PoolModel(10, 2)
    a = pool.seq_create()
    pool.append_slots([a], [3])
    b, c = pool.fork(a), pool.fork(a)
    shared_last = pool.tables[a][-1]
    assert pool.ref[shared_last] == 3
    slots, cow = pool.append_slots([a, b, c], [1, 1, 1])
    assert len(cow) == 2
    assert all(src == shared_last for src, _ in cow)
    assert pool.tables[c][-1] == shared_last       # last sharer keeps the block
    assert pool.ref[shared_last] == 1
    assert pool.tables[a][0] == pool.tables[b][0] == pool.tables[c][0]
    assert pool.ref[pool.tables[a][0]] == 3        # full shared block never copied
    assert len(set(slots)) == 3
    pool.check_invariants()


def test_full_shared_block_is_not_copied():
    pool = PoolModel(10, 2)
    a = pool.seq_create()
    pool.append_slots([a], [4])
    b = pool.fork(a)
    _, cow = pool.append_slots([a, b], [1, 1])
    assert cow == []
    pool.check_invariants()


def test_exhaustion_changes_nothing():
    pool = PoolModel(3, 2)
    a, b = pool.seq_create(), pool.seq_create()
    pool.append_slots([a], [3])
    before = (pool.export(), {k: list(v) for k, v in pool.tables.items()}, dict(pool.lengths))
    with pytest.raises(NoBlocks):
        pool.append_slots([a, b], [1, 3])          # needs 2 blocks, 1 is free
    after = (pool.export(), {k: list(v) for k, v in pool.tables.items()}, dict(pool.lengths))
    assert before == after


def test_free_returns_blocks_to_tail_in_logical_order():
    pool = PoolModel(6, 1, free_order=[4, 1, 5, 0, 2, 3])
    a = pool.seq_create()
    pool.append_slots([a], [3])                    # takes 4, 1, 5
    pool.free_seq(a)
    assert list(pool.free) == [0, 2, 3, 4, 1, 5]
    with pytest.raises(BadSeq):
        pool.free_seq(a)


def test_set_table_errors():
    pool = PoolModel(4, 2)
    a = pool.seq_create()
    with pytest.raises(InvalidArg):
        pool.set_table(a, [0, 1], 5)               # 5 tokens need 3 pages
    with pytest.raises(InvalidArg):
        pool.set_table(a, [0, 7], 4)               # block outside the pool
    pool.set_table(a, [0, 1], 4)
    b = pool.seq_create()
    with pytest.raises(InvalidArg):
        pool.set_table(b, [1], 2)                  # block already in use


def test_unshared_slots_are_disjoint_and_cover_the_blocks():
    rng = random.Random(3)
    pool = PoolModel(64, 4, free_order=rng.sample(range(64), 64))
    seqs = [pool.seq_create() for _ in range(6)]
    for _ in range(30):
        sid = rng.choice(seqs)
        pool.append_slots([sid], [rng.randint(0, 3)])
    all_slots = []
    for sid in seqs:
        s = pool.slots_of(sid)
        assert len(s) == pool.lengths[sid]
        held = {x for blk in pool.tables[sid] for x in range(blk * 4, blk * 4 + 4)}
        assert set(s) <= held
        all_slots += s
    assert len(all_slots) == len(set(all_slots))


@settings(max_examples=60, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 4), st.integers(0, 7), st.integers(0, 5)),
                min_size=1, max_size=40),
       st.integers(1, 4), st.integers(0, 10 ** 6))
def test_invariants_under_random_operations(ops, page, seed):
    rng = random.Random(seed)
    nb = 24
    pool = PoolModel(nb, page, free_order=rng.sample(range(nb), nb))
    live = []
    for kind, pick, n in ops:
        try:
            if kind == 0 or not live:
                live.append(pool.seq_create())
            elif kind == 1:
                sids = list(dict.fromkeys(live[(pick + i) % len(live)] for i in range(1 + n % 3)))
                pool.append_slots(sids, [n] * len(sids))
            elif kind == 2:
                live.append(pool.fork(live[pick % len(live)]))
            elif kind == 3:
                pool.free_seq(live.pop(pick % len(live)))
            else:
                pool.append_slots([live[pick % len(live)]], [1])
        except NoBlocks:
            pass
        pool.check_invariants()
        st_ = pool.stats()
        assert st_["free_blocks"] + st_["used_blocks"] == nb
        assert 0 <= st_["wasted_slots"] <= st_["used_blocks"] * page
        # a shared block is counted once: live tokens never exceed slots in use
        assert st_["live_tokens"] <= st_["allocated_slots"]


def test_layout_round_trip_through_printed_table(golden):
    import numpy as np
    phys = golden("block_table_example.json")["physical_blocks"]
    page, hkv, d = 2, 2, 3
    kc = np.zeros((16, hkv, page, d), np.float32)
    vc = np.zeros((16, hkv, d, page), np.float32)
    length = 5
    k = np.arange(length * hkv * d, dtype=np.float32).reshape(length, hkv, d) + 1
    v = -k
    slots = [layout.slot_of(phys, page, t) for t in range(length)]
    layout.write_tokens(kc, vc, slots, k, v)
    assert (kc[8, :, 0, :] == k[0]).all() and (kc[3, :, 1, :] == k[3]).all()
    assert (vc[11, :, :, 0] == v[4]).all()
    k2, v2 = layout.read_sequence(kc, vc, phys, length)
    assert (k2 == k).all() and (v2 == v).all()
    untouched = [b for b in range(16) if b not in phys]
    assert (kc[untouched] == 0).all() and (vc[untouched] == 0).all()
