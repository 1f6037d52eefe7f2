"""Fragmentation accounting: fixed reservation vs paged allocation.

Source: the "inference-acceleration-pagedattention-vllm" chapter (the
fragmentation demo and its worked example), with the lengths / reservation /
page-size symbols whose glyphs were lost read as L_i, R and P.  The
"PagedAttention Internals" lesson ("The Memory Waste Problem", "Fixed-Size KV
Blocks") and the "pagedattention" topic page (second and third paragraphs and
the comparison table) describe the same two schemes in prose.

Definitions used here (the chapter's formulas did not survive extraction; this
is the plainest reading that reproduces its printed numbers):

* naive:  every sequence holds a fixed reservation of R slots, whatever its
          length (requires L_i <= R);
* paged:  a sequence holds whole pages only, ceil(L_i / P) of them;
* wasted = allocated - used;  fragmentation = wasted / allocated, where the
  denominator is the allocated slots, not the whole pool.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict, Iterable


def _check_lengths(lengths: Iterable[int]):
    ls = [int(x) for x in lengths]
    if any(x < 0 for x in ls):
        raise ValueError("negative length")
    return ls


def summarize(allocated: int, used: int) -> Dict[str, object]:
    """Allocated / used / wasted slots and the fragmentation fraction."""
    if used > allocated:
        raise ValueError("more tokens than allocated slots")
    wasted = allocated - used
    frac = Fraction(wasted, allocated) if allocated else Fraction(0)
    return {"allocated": allocated, "used": used, "wasted": wasted,
            "fragmentation": frac}


def naive(lengths: Iterable[int], reservation: int) -> Dict[str, object]:
    """Fixed per-sequence reservation of ``reservation`` slots."""
    ls = _check_lengths(lengths)
    if any(x > reservation for x in ls):
        raise ValueError("a sequence outgrew its reservation")
    return summarize(reservation * len(ls), sum(ls))


def pages_needed(length: int, page: int) -> int:
    """Whole pages a sequence of ``length`` tokens holds: ceil(length / page)."""
    if page <= 0:
        raise ValueError("page size must be positive")
    return -(-int(length) // int(page))


def paged(lengths: Iterable[int], page: int) -> Dict[str, object]:
    """Page-by-page allocation with pages of ``page`` slots, nothing shared."""
    ls = _check_lengths(lengths)
    return summarize(sum(page * pages_needed(x, page) for x in ls), sum(ls))


def paged_waste(length: int, page: int) -> int:
    """Slots wasted by one sequence: those of its partly filled last page."""
    return page * pages_needed(length, page) - int(length)
