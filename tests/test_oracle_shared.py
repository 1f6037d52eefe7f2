"""Pins for oracle.layout.shared_prefix_tokens (tokens two sequences hold in the same slots).

A fork points at every block of its parent ("pagedattention" topic page,
fourth paragraph), so right after a fork the two share the whole context; a
write into a shared partial block copies it first ("PagedAttention
Internals", "Sharing And Dynamic Growth"), after which only the whole blocks
before it are shared.  These closed forms come from the pool model's
behaviour, not from the oracle function's token loop.
"""
import numpy as np
import pytest

from oracle import layout as olayout
from oracle.pool_model import PoolModel


def _shared(pm, a, b):
    return olayout.shared_prefix_tokens(pm.tables[a], pm.lengths[a], pm.tables[b], pm.lengths[b],
                                        pm.block_size)


@pytest.mark.parametrize("p,length", [(1, 5), (2, 3), (4, 8), (16, 37), (16, 32)])
def test_fork_shares_everything_then_copy_on_write_keeps_whole_blocks(p, length):
    pm = PoolModel(64, p)
    root = pm.seq_create()
    pm.append_slots([root], [length])
    kids = [pm.fork(root) for _ in range(3)]
    for k in kids:
        assert _shared(pm, root, k) == length
        assert _shared(pm, k, root) == length
    # one more token each, in call order: sharers of a partial last block copy it
    pm.append_slots([root] + kids, [1, 1, 1, 1])
    whole = length - length % p
    want = length if length % p == 0 else whole
    for a in [root] + kids:
        for b in [root] + kids:
            if a != b:
                assert _shared(pm, a, b) == want
    # a sequence with itself shares its whole length
    assert _shared(pm, root, root) == length + 1


def test_unrelated_sequences_share_nothing():
    pm = PoolModel(16, 4)
    a, b = pm.seq_create(), pm.seq_create()
    pm.append_slots([a, b], [9, 7])
    assert _shared(pm, a, b) == 0
    empty = pm.seq_create()
    assert _shared(pm, a, empty) == 0


def test_printed_block_table_with_a_diverging_third_block():
    """The table 8, 3, 11 ("The Block Table Map") against 8, 3, 5 at P = 2:
    two whole blocks (4 tokens) in common, limited by the shorter length."""
    t1, t2 = [8, 3, 11], [8, 3, 5]
    assert olayout.shared_prefix_tokens(t1, 6, t2, 6, 2) == 4
    assert olayout.shared_prefix_tokens(t1, 6, t2, 3, 2) == 3
    assert olayout.shared_prefix_tokens(t1, 1, t2, 6, 2) == 1
    assert olayout.shared_prefix_tokens([8, 3, 11], 6, [9, 3, 11], 6, 2) == 0


def test_random_tables_match_whole_block_count():
    """Brute force on small random tables: the token-by-token count equals the
    number of leading equal block ids times P, capped by both lengths."""
    rng = np.random.default_rng(11)
    for _ in range(400):
        p = int(rng.choice([1, 2, 3, 4, 8]))
        n = int(rng.integers(0, 6))
        base = rng.integers(0, 5, size=n).tolist()
        other = list(base)
        if n and rng.random() < 0.7:
            j = int(rng.integers(0, n))
            other[j] = (other[j] + 1 + int(rng.integers(0, 3))) % 7
        la = int(rng.integers(0, n * p + 1))
        lb = int(rng.integers(0, n * p + 1))
        k = 0
        while k < n and base[k] == other[k]:
            k += 1
        assert olayout.shared_prefix_tokens(base, la, other, lb, p) == min(k * p, la, lb)
