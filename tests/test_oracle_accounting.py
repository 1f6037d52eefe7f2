"""Pins of the oracle's fragmentation accounting to the pages' printed numbers."""
from fractions import Fraction

import pytest

from oracle import accounting
from oracle.pool_model import PoolModel


def test_naive_worked_example(golden):
    ex = golden("fragmentation_examples.json")["naive_reservation"]
    r = accounting.naive(ex["lengths"], ex["reservation"])
    assert r["used"] == ex["used"]
    assert r["allocated"] == ex["allocated"]
    assert r["wasted"] == ex["wasted"]
    assert round(float(r["fragmentation"]), 3) == ex["fragmentation_3dp"]


def test_paged_worked_example(golden):
    ex = golden("fragmentation_examples.json")["paged_page2"]
    r = accounting.paged(ex["lengths"], ex["page"])
    assert r["used"] == ex["used"]
    assert r["wasted"] == ex["wasted"]            # printed: only one slot wasted
    assert r["allocated"] == ex["allocated"]      # reconstructed from it
    assert r["fragmentation"] == Fraction(1, 8)
    assert float(r["fragmentation"]) == ex["fragmentation"]


def test_worked_example_pool_model_token_by_token(golden):
    """The pool model, fed one token at a time, lands on the printed waste.

    This pins lazy allocation: taking a block when the previous one fills
    (rather than when the next token arrives) would hold 12 slots, not 8.
    """
    ex = golden("fragmentation_examples.json")["paged_page2"]
    pool = PoolModel(16, ex["page"])
    seqs = [pool.seq_create() for _ in ex["lengths"]]
    for sid, n in zip(seqs, ex["lengths"]):
        for _ in range(n):
            pool.append_slots([sid], [1])
    st = pool.stats()
    assert st["allocated_slots"] == ex["allocated"]
    assert st["wasted_slots"] == ex["wasted"]
    assert st["live_tokens"] == ex["used"]
    assert st["fragmentation"] == ex["fragmentation"]


def test_exercise_two_arrivals(golden):
    ex = golden("fragmentation_examples.json")["exercise_arrivals"]
    r = accounting.paged(ex["lengths"], ex["page"])
    assert (r["allocated"], r["wasted"]) == (ex["allocated"], ex["wasted"])
    # together with the worked example's three sequences
    both = accounting.paged([1, 4, 2] + ex["lengths"], ex["page"])
    assert (both["allocated"], both["wasted"]) == (14, 3)


def test_long_reservation_example(golden):
    ex = golden("fragmentation_examples.json")["long_reservation"]
    naive = accounting.naive([ex["length"]], ex["reservation"])
    assert naive["wasted"] == ex["reservation"] - ex["length"]
    assert naive["fragmentation"] == Fraction(9, 10)
    p16 = accounting.paged([ex["length"]], 16)
    assert (p16["allocated"], p16["wasted"]) == (208, 8)
    assert float(p16["fragmentation"]) < 0.05      # "a few percent"


def test_naive_reservation_ignores_length():
    for n in range(0, 9):
        assert accounting.naive([n], 8)["allocated"] == 8
    with pytest.raises(ValueError):
        accounting.naive([9], 8)


def test_paged_waste_bound_brute_force():
    """Waste counted slot by slot equals the closed form and stays below a page."""
    for page in range(1, 33):
        for length in range(0, 65):
            slots = 0
            for t in range(length):          # a page is taken when a token needs one
                if t % page == 0:
                    slots += page
            waste = slots - length
            assert waste == accounting.paged_waste(length, page)
            assert 0 <= waste <= page - 1
            assert accounting.paged([length], page)["wasted"] == waste


def test_total_paged_waste_below_one_page_per_sequence():
    lengths = [1, 17, 33, 200, 4096, 5]
    for page in (2, 8, 16, 32):
        r = accounting.paged(lengths, page)
        assert r["wasted"] < len(lengths) * page
