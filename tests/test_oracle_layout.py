"""Pins for oracle.layout's token-major key order.

The key cache may hold a block's rows head by head ([P, D] per head) or token
by token ([Hkv, D] per token).  The second is the first with the head and
token axes of every block swapped, which numpy's transpose states
independently of the element loop in the oracle.
"""
import numpy as np
import pytest

from oracle import layout as olayout
def test_token_major_keys_are_the_head_major_cache_transposed():
    """Writing with the token-major key order equals writing head-major and then
    swapping the head and token axes of every block (numpy's transpose)."""
    rng = np.random.default_rng(3)
    nb, hkv, p, d, n = 6, 3, 4, 5, 17
    slots = rng.choice(nb * p, size=n, replace=False)
    slots[4] = -1
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    kh, vh = np.zeros((nb, hkv, p, d)), np.zeros((nb, hkv, d, p))
    kt, vt = np.zeros((nb, p, hkv, d)), np.zeros((nb, hkv, d, p))
    olayout.write_tokens(kh, vh, slots, k, v)
    olayout.write_tokens(kt, vt, slots, k, v, token_major=True)
    assert np.array_equal(kt, np.transpose(kh, (0, 2, 1, 3)))
    assert np.array_equal(vt, vh)
    table = [int(s) // p for s in slots[:3]]
    a = olayout.read_sequence(kh, vh, table, 3 * p)
    b = olayout.read_sequence(kt, vt, table, 3 * p, token_major=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# copy_block: the cache side of copy-on-write.  Forked sequences point at the
# same blocks, and a sharer that writes into a shared, partly filled block gets
# a private copy first ("pagedattention" topic page, fourth paragraph and the
# comparison table's sharing row; "PagedAttention Internals", "Sharing And
# Dynamic Growth").  The pin is the observable contract, not the two
# assignments: after the pool model's copy-on-write pairs are applied with
# copy_block and every sharer's new token is written, each sharer reads back
# exactly the tokens it was given (the common prefix plus its own), and blocks
# nothing touched keep their fill.  Planted mistakes in the copy (source and
# destination swapped, keys only, values only, one head only) must each
# break that contract.
# ---------------------------------------------------------------------------
from oracle.pool_model import PoolModel  # noqa: E402

FILL = -7.0


def _copy_swapped(k_cache, v_cache, src, dst):
    olayout.copy_block(k_cache, v_cache, dst, src)


def _copy_keys_only(k_cache, v_cache, src, dst):
    k_cache[dst] = k_cache[src]


def _copy_values_only(k_cache, v_cache, src, dst):
    v_cache[dst] = v_cache[src]


def _copy_first_head_only(k_cache, v_cache, src, dst):
    k_cache[dst, 0] = k_cache[src, 0]
    v_cache[dst, 0] = v_cache[src, 0]


def _fan_out_story(copy, token_major=False, prefix=3, page=2, sharers=3, hkv=2, d=4, nb=10):
    """Prefix of `prefix` tokens, forked into `sharers` sequences that append one
    token each.  Returns (k_cache, v_cache, model, seq ids, expected K/V per seq,
    the blocks no sequence holds, number of copies)."""
    rng = np.random.default_rng(11)
    pm = PoolModel(nb, page)
    root = pm.seq_create()
    shape_k = (nb, page, hkv, d) if token_major else (nb, hkv, page, d)
    k_cache = np.full(shape_k, FILL)
    v_cache = np.full((nb, hkv, d, page), FILL)
    pk, pv = rng.standard_normal((prefix, hkv, d)), rng.standard_normal((prefix, hkv, d))
    slots, cow = pm.append_slots([root], [prefix])
    assert cow == []
    olayout.write_tokens(k_cache, v_cache, slots, pk, pv, token_major)
    seqs = [root] + [pm.fork(root) for _ in range(sharers - 1)]
    nk, nv = rng.standard_normal((sharers, hkv, d)), rng.standard_normal((sharers, hkv, d))
    slots, cow = pm.append_slots(seqs, [1] * sharers)
    for src, dst in cow:
        copy(k_cache, v_cache, src, dst)
    olayout.write_tokens(k_cache, v_cache, slots, nk, nv, token_major)
    want = {s: (np.concatenate([pk, nk[i:i + 1]]), np.concatenate([pv, nv[i:i + 1]]))
            for i, s in enumerate(seqs)}
    held = {b for s in seqs for b in pm.tables[s]}
    untouched = [b for b in range(nb) if b not in held]
    return k_cache, v_cache, pm, seqs, want, untouched, len(cow)


def _contract_holds(k_cache, v_cache, pm, seqs, want, untouched, token_major=False):
    for s in seqs:
        k, v = olayout.read_sequence(k_cache, v_cache, pm.tables[s], pm.lengths[s], token_major)
        if not (np.array_equal(k, want[s][0]) and np.array_equal(v, want[s][1])):
            return False
    return all(np.all(k_cache[b] == FILL) and np.all(v_cache[b] == FILL) for b in untouched)


@pytest.mark.parametrize("token_major", [False, True])
def test_copy_on_write_each_sharer_reads_its_own_tokens(token_major):
    """Prefix of 3 tokens in pages of 2, three sharers: the shared partial block
    is copied twice (the last sharer writes in place), and every sharer then
    reads the prefix followed by its own token."""
    k, v, pm, seqs, want, untouched, ncopies = _fan_out_story(olayout.copy_block, token_major)
    assert ncopies == 2
    assert _contract_holds(k, v, pm, seqs, want, untouched, token_major)
    # the whole first block stays shared by all three, untouched by the copies
    assert len({pm.tables[s][0] for s in seqs}) == 1
    assert len({pm.tables[s][1] for s in seqs}) == 3


@pytest.mark.parametrize("mutant", [_copy_swapped, _copy_keys_only, _copy_values_only,
                                    _copy_first_head_only])
@pytest.mark.parametrize("token_major", [False, True])
def test_copy_on_write_planted_mistakes_break_the_contract(mutant, token_major):
    k, v, pm, seqs, want, untouched, _ = _fan_out_story(mutant, token_major)
    assert not _contract_holds(k, v, pm, seqs, want, untouched, token_major)


def test_copy_block_moves_every_slot_of_the_block_and_nothing_else():
    """Brute force over every element: after one copy the destination block
    equals the source block element for element, and every other block is
    unchanged."""
    rng = np.random.default_rng(5)
    for token_major in (False, True):
        nb, p, hkv, d = 5, 3, 2, 4
        k = rng.standard_normal((nb, p, hkv, d) if token_major else (nb, hkv, p, d))
        v = rng.standard_normal((nb, hkv, d, p))
        k0, v0 = k.copy(), v.copy()
        olayout.copy_block(k, v, 1, 3)
        for b in range(nb):
            for idx in np.ndindex(k.shape[1:]):
                assert k[(b,) + idx] == (k0[(1,) + idx] if b == 3 else k0[(b,) + idx])
            for idx in np.ndindex(v.shape[1:]):
                assert v[(b,) + idx] == (v0[(1,) + idx] if b == 3 else v0[(b,) + idx])
