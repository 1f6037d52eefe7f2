"""Pins for oracle.layout's token-major key order.

The key cache may hold a block's rows head by head ([P, D] per head) or token
by token ([Hkv, D] per token).  The second is the first with the head and
token axes of every block swapped, which numpy's transpose states
independently of the element loop in the oracle.
"""
import numpy as np

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
