"""Slots and the expected contents of the paged K / V caches.

Source: "PagedAttention Internals", sections "Paging Comes From Operating
Systems" and "The Block Table Map" (logical order is kept by the table while
the physical blocks sit anywhere), and the "pagedattention" topic page, third
paragraph (logical block N may live in any free physical block).

The pages fix no memory layout.  The layout read here, which the GPU library
also uses, is:

* ``k_cache[num_blocks, num_kv_heads, P, D]``: token ``o`` of block ``blk``,
  head ``h``, is the row ``k_cache[blk, h, o, :]``;
* ``v_cache[num_blocks, num_kv_heads, D, P]``: the same token's value vector is
  the column ``v_cache[blk, h, :, o]`` (each block stores its values
  transposed);
* with ``token_major=True`` the key cache is ``k_cache[num_blocks, P,
  num_kv_heads, D]`` instead (all heads of one token together), the row
  ``k_cache[blk, o, h, :]``; values are unchanged;

and slot ``s`` means block ``s // P``, offset ``s % P``.  A negative slot means
"do not write".  Arrays are copied bit for bit (uint16 patterns for bf16).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def slot_of(table: Sequence[int], block_size: int, t: int) -> int:
    """Slot holding logical token ``t`` of a sequence with this block table."""
    return int(table[t // block_size]) * block_size + t % block_size


def _shape(k_cache, v_cache, token_major):
    nb, hkv, d, p = v_cache.shape
    assert k_cache.shape == ((nb, p, hkv, d) if token_major else (nb, hkv, p, d))
    return nb, hkv, p, d


def write_tokens(k_cache: np.ndarray, v_cache: np.ndarray, slots: Sequence[int],
                 k: np.ndarray, v: np.ndarray, token_major: bool = False) -> None:
    """Store token i's K/V (``k[i]``, ``v[i]`` of shape [Hkv, D]) at ``slots[i]``."""
    nb, hkv, p, d = _shape(k_cache, v_cache, token_major)
    assert k.shape == v.shape == (len(slots), hkv, d)
    for i, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = divmod(s, p)
        for h in range(hkv):
            if token_major:
                k_cache[blk, off, h, :] = k[i, h, :]
            else:
                k_cache[blk, h, off, :] = k[i, h, :]
            v_cache[blk, h, :, off] = v[i, h, :]


def read_sequence(k_cache: np.ndarray, v_cache: np.ndarray, table: Sequence[int],
                  length: int, token_major: bool = False):
    """Gather a sequence's K/V back into logical order: ([L,Hkv,D], [L,Hkv,D])."""
    nb, hkv, p, d = _shape(k_cache, v_cache, token_major)
    ks = np.empty((length, hkv, d), dtype=k_cache.dtype)
    vs = np.empty((length, hkv, d), dtype=v_cache.dtype)
    for t in range(length):
        blk, off = divmod(slot_of(table, p, t), p)
        ks[t] = k_cache[blk, off, :, :] if token_major else k_cache[blk, :, off, :]
        vs[t] = v_cache[blk, :, :, off]
    return ks, vs


def copy_block(k_cache: np.ndarray, v_cache: np.ndarray, src: int, dst: int) -> None:
    """Copy-on-write: every slot of block ``src`` (all heads, K and V) to ``dst``."""
    k_cache[dst] = k_cache[src]
    v_cache[dst] = v_cache[src]


def shared_prefix_tokens(table_a: Sequence[int], len_a: int, table_b: Sequence[int], len_b: int,
                         block_size: int) -> int:
    """How many leading tokens two sequences hold in the very same slots.

    Source: "pagedattention" topic page, fourth paragraph, and "PagedAttention
    Internals", "Sharing And Dynamic Growth": forked sequences point at the
    same physical blocks until one of them writes.  Read here as the largest
    n <= min(len_a, len_b) such that every logical token t < n has the same
    slot in both sequences, found token by token; tokens in the same slot are
    the same bytes, so attention may read them once for both.
    """
    n = 0
    while n < min(len_a, len_b) and \
            slot_of(table_a, block_size, n) == slot_of(table_b, block_size, n):
        n += 1
    return n
