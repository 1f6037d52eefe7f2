"""Incremental block-table uploads against full uploads, bit for bit.

An incrementally patched device table, its lengths and its slot mapping must
equal what a full upload of the same pool state writes, after every kind of
change the pool makes: tokens appended within a block and across block
boundaries, copy-on-write replacing a table entry, a row that starts holding
another sequence, rows added, and a patch too large for kernel arguments
(which falls back to the full upload).
"""
import numpy as np
import pytest

from tests.paged_case import say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_guard(request):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"\n[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()


def _upload_pair(pool, seqs, max_blocks, inc, slots=None):
    """Incremental upload into the tracked buffers `inc`, full upload into fresh ones."""
    import torch
    table = torch.full((len(seqs), max_blocks), 12345, dtype=torch.int32, device="cuda")
    lens = torch.full((len(seqs),), -7, dtype=torch.int32, device="cuda")
    dslots = None
    if slots is not None:
        dslots = torch.full((max(len(slots), 1),), -9, dtype=torch.int32, device="cuda")
    r_full = pool.block_table_upload(seqs, max_blocks, table, lens, slots, dslots)
    r_inc = pool.block_table_upload(seqs, max_blocks, inc["table"], inc["lens"], slots,
                                    inc.get("slots"), incremental=True)
    torch.cuda.synchronize()
    assert r_full == r_inc
    n = len(seqs)
    assert torch.equal(inc["table"][:n], table), "incremental table differs from the full upload"
    assert torch.equal(inc["lens"][:n], lens)
    if slots is not None:
        assert torch.equal(inc["slots"][:len(slots)], dslots[:len(slots)])
    # every row: the pool's own table, then -1
    for i, s in enumerate(seqs):
        t, ln = pool.get_table(s)
        row = table[i].cpu().numpy()
        assert np.array_equal(row[:len(t)], t) and (row[len(t):] == -1).all()
        assert lens[i].item() == ln


def test_incremental_upload_tracks_every_change():
    import torch
    from paged_kv_cache_399_amd import BlockPool
    rng = np.random.default_rng(11)
    nb, p, mb = 4096, 16, 96
    pool = BlockPool(nb, p, rng.permutation(nb))
    seqs = [pool.seq_create() for _ in range(24)]
    pool.append_slots(seqs, rng.integers(1, 400, size=len(seqs)))
    inc = {"table": torch.empty((40, mb), dtype=torch.int32, device="cuda"),
           "lens": torch.empty(40, dtype=torch.int32, device="cuda"),
           "slots": torch.empty(64, dtype=torch.int32, device="cuda")}
    # first upload into a new table: the incremental flag falls back to a full upload
    _upload_pair(pool, seqs, mb, inc)
    for step in range(30):
        # one decode token each, with the slot mapping riding along
        slots, cow = pool.append_slots(seqs, np.ones(len(seqs), np.int32))
        assert len(cow) == 0
        _upload_pair(pool, seqs, mb, inc, slots)
    # several tokens at once across block boundaries
    pool.append_slots(seqs, rng.integers(0, 40, size=len(seqs)))
    _upload_pair(pool, seqs, mb, inc)
    # copy-on-write: fork row 3's sequence into row 5's place, then both diverge
    parent = seqs[3]
    if pool.get_table(parent)[1] % p == 0:
        pool.append_slots([parent], [1])
    child = pool.fork(parent)
    seqs[5] = child
    _, cow = pool.append_slots([parent, child], [1, 1])
    assert len(cow) == 1                                  # the partial block was copied once
    _upload_pair(pool, seqs, mb, inc)
    # a freed sequence's row is taken by a new one; rows are added at the end
    pool.free(seqs[7])
    seqs[7] = pool.seq_create()
    pool.append_slots([seqs[7]], [33])
    seqs += [pool.seq_create() for _ in range(6)]
    pool.append_slots(seqs[-6:], [1, 16, 17, 200, 5, 64])
    _upload_pair(pool, seqs, mb, inc)
    # rows dropped from the end, then a decode step
    seqs = seqs[:20]
    slots, _ = pool.append_slots(seqs, np.ones(len(seqs), np.int32))
    _upload_pair(pool, seqs, mb, inc, slots)


def test_large_patch_falls_back_to_full_upload():
    import torch
    from paged_kv_cache_399_amd import BlockPool
    nb, p, mb = 65536, 8, 700
    pool = BlockPool(nb, p)
    seqs = [pool.seq_create() for _ in range(64)]
    pool.append_slots(seqs, [10] * 64)
    inc = {"table": torch.empty((64, mb), dtype=torch.int32, device="cuda"),
           "lens": torch.empty(64, dtype=torch.int32, device="cuda")}
    _upload_pair(pool, seqs, mb, inc)
    # 64 sequences x ~600 new blocks: far more than the kernel-argument patches carry
    pool.append_slots(seqs, [4800] * 64)
    _upload_pair(pool, seqs, mb, inc)
    pool.append_slots(seqs, [1] * 64)
    _upload_pair(pool, seqs, mb, inc)
