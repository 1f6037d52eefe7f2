"""Pins for oracle.admission: closed forms, a hand-traced example, invariants.

The loop is the reading stated in the module (admit while the queue head fits,
one token per running sequence, most recently admitted preempted first when
blocks run out, release on finish).  Its results are fixed here by arithmetic
done outside the code: whole-batch closed forms for identical requests, a
four-step trace worked by hand, and identities every replay must satisfy.
"""
import math

import numpy as np
import pytest

from oracle import admission as oad
from synth import ADMISSION_CONFIGS, make_admission_trace


@pytest.mark.parametrize("a,b,m,cap,n", [(10, 5, 20, 100, 7), (1, 1, 1, 2, 5), (30, 7, 70, 1000, 33)])
def test_reserved_identical_requests_closed_form(a, b, m, cap, n):
    """k = cap // (a + m) run together; each wave of k runs b steps."""
    out = oad.reserved(cap, [a] * n, [b] * n, [m] * n)
    k = cap // (a + m)
    waves = math.ceil(n / k)
    rec = out["rec"]
    assert len(rec["running"]) == waves * b
    expect = []
    for w in range(waves):
        expect += [min(k, n - w * k)] * b
    assert rec["running"] == expect
    assert out["completed"] == n


@pytest.mark.parametrize("x,p,nb,n", [(3, 16, 10, 7), (1, 4, 5, 12), (2, 8, 64, 100)])
def test_paged_requests_filling_whole_blocks_closed_form(x, p, nb, n):
    """Prompt x P - 1 and one output token: every request holds exactly x blocks,
    never grows past them, so nb // x run per step and nothing is preempted."""
    a = x * p - 1
    out = oad.paged(nb, p, [a] * n, [1] * n)
    k = nb // x
    rec = out["rec"]
    assert rec["running"] == [min(k, n - s * k) for s in range(math.ceil(n / k))]
    assert sum(rec["preempted"]) == 0
    # every request finishes in the step it starts, so nothing is held after a step
    assert all(h == 0 for h in rec["held"])
    assert out["completed"] == n


def test_paged_hand_traced_preemption_example():
    """3 blocks of 2 slots; requests (prompt, output) = (1, 3), (2, 2), (1, 1).

    Step 1: all three fit at admission (1 + 2 + 1 blocks needed: 1, 2, 1 free
    in turn); r1's token opens a new block but none is free, so r2 (admitted
    last) is preempted.  Step 2: r0 now opens a block, r1 is preempted.
    Step 3: r1 would need 2 blocks (context 3 + 1), only 1 is free; r0
    finishes.  Step 4: r1 and r2 are readmitted and both finish.
    """
    out = oad.paged(3, 2, [1, 2, 1], [3, 2, 1])
    rec = out["rec"]
    assert rec["running"] == [2, 1, 1, 2]
    assert rec["held"] == [6, 4, 0, 0]
    assert rec["live"] == [5, 3, 0, 0]
    assert rec["admitted"] == [3, 0, 0, 2]
    assert rec["finished"] == [0, 0, 1, 2]
    assert rec["preempted"] == [1, 1, 0, 0]


def test_reserved_hand_traced_example():
    """Capacity 6, reservations prompt + 4 = 5, 6, 5: one request at a time."""
    out = oad.reserved(6, [1, 2, 1], [3, 2, 1], [4, 4, 4])
    rec = out["rec"]
    assert rec["running"] == [1, 1, 1, 1, 1, 1]
    assert rec["held"] == [5, 5, 0, 6, 0, 0]
    assert rec["live"] == [2, 3, 0, 3, 0, 0]
    assert rec["admitted"] == [1, 0, 0, 1, 0, 1]
    assert rec["finished"] == [0, 0, 1, 0, 1, 1]


def test_requests_that_never_fit_are_rejected():
    out = oad.paged(4, 4, [10, 20, 3], [6, 1, 1])       # 16 slots: 10 + 6 fits, 20 + 1 does not
    assert out["rejected"] == [1] and out["completed"] == 2
    out = oad.reserved(16, [10, 3], [2, 2], [7, 13])    # 17 > 16, 16 fits
    assert out["rejected"] == [0] and out["completed"] == 1


def test_invariants_on_a_synthetic_trace():
    cfg = ADMISSION_CONFIGS["admission_small"]
    pr, ou, mx, fo = make_admission_trace(cfg, 3)
    p, nb = cfg.block_size, cfg.num_blocks
    pg = oad.paged(nb, p, pr, ou, fo)
    rs = oad.reserved(nb * p, pr, ou, mx)
    for out in (pg, rs):
        rec = out["rec"]
        # every output token is generated exactly once, preemption or not
        assert sum(rec["running"]) == int(ou.sum())
        assert out["completed"] == len(pr) and not out["rejected"]
        assert all(0 <= l <= h <= nb * p for l, h in zip(rec["live"], rec["held"]))
        assert sum(rec["admitted"]) == len(pr) + sum(rec["preempted"])
    # paged: a resident sequence wastes less than one block
    resident = np.cumsum(np.asarray(pg["rec"]["admitted"]) - np.asarray(pg["rec"]["preempted"])
                         - np.asarray(pg["rec"]["finished"]))
    waste = np.asarray(pg["rec"]["held"]) - np.asarray(pg["rec"]["live"])
    assert np.all(waste <= (p - 1) * resident)
    assert sum(pg["rec"]["preempted"]) > 0           # the trace exercises preemption
    # the reservation holds prompt + limit for each resident request
    assert np.mean(rs["rec"]["running"]) < np.mean(pg["rec"]["running"])


def test_paged_admission_needs_room_for_the_next_token():
    """2 blocks of 2 slots; requests (1, 3), (2, 1).  r1's context of 2 fills
    one block exactly, so its first token needs a second block: it waits until
    r0 finishes (step 3) and runs in step 4.
    """
    rec = oad.paged(2, 2, [1, 2], [3, 1])["rec"]
    assert rec["running"] == [1, 1, 1, 1]
    assert rec["held"] == [2, 4, 0, 0]
    assert rec["live"] == [2, 3, 0, 0]
    assert rec["admitted"] == [1, 0, 0, 1]
    assert rec["finished"] == [0, 0, 1, 1]
    assert rec["preempted"] == [0, 0, 0, 0]


def test_planted_mistake_is_caught():
    """An oracle that forgets the next token at admission admits r1 in step 1
    of the example above and then has to preempt it: the pinned records differ."""
    saved = oad._blocks
    try:
        oad._blocks = lambda t, p: (t - 1 + p - 1) // p
        rec = oad.paged(2, 2, [1, 2], [3, 1])["rec"]
    finally:
        oad._blocks = saved
    assert rec["admitted"][0] == 2 and rec["preempted"][0] == 1
    assert rec["admitted"] != [1, 0, 0, 1]
