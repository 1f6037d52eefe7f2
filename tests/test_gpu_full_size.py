"""Parity at the full benchmark sizes, in the launch configuration bench.py times.

Each decode workload is built exactly as bench.py builds it: same seed, pool
size and order, bulk append, and batch metadata and workspace sized for
bench.py's default warm-up plus timed steps (so the same partition length and
grid).  One decode step then runs through the library, and every part of it is
compared with the oracle, for every sequence:

* allocator state after the bulk append and again after the decode append:
  the slot of every token, every block table (the pool's and the padded device
  copy the kernels read), every length, the free list in order, every
  refcount, and the device's shared-token counts ("PagedAttention Internals",
  "Fixed-Size KV Blocks" and "The Block Table Map");
* the cache: every sequence's keys and values, gathered through the oracle
  model's tables with the oracle layout, equal the generated ones bit for bit;
* attention: every sequence's output within 2e-2 of float64.

Prefill workloads: every new token's output against the float64 causal oracle
and every sequence's cache rows bit for bit.
"""
import numpy as np
import pytest

import bench
from oracle import attention as oatt
from oracle import layout as olayout
from oracle.pool_model import PoolModel
from synth import CONFIGS, PREFILL_CONFIGS, make_prefill_workload, make_workload
from tests.paged_case import BF16_TOL, host_bits, say

pytestmark = pytest.mark.gpu

BENCH_STEPS = bench.DEFAULT_WARMUP + bench.DEFAULT_STEPS   # sizes the batch metadata


@pytest.fixture(autouse=True)
def _gpu_guard(request):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"\n[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()
    import paged_kv_cache_399_amd as pkv
    assert pkv.check_device_errors() == 0


def _cache_rows(kv, table, length):
    """(k, v) host bits of one sequence in logical order: its blocks (taken from
    the oracle model's table) copied from the device cache, then gathered with
    the oracle layout."""
    import torch
    idx = torch.from_numpy(np.asarray(table, np.int64)).to(kv.k_cache.device)
    kc = host_bits(kv.k_cache.index_select(0, idx))
    vc = host_bits(kv.v_cache.index_select(0, idx))
    return olayout.read_sequence(kc, vc, list(range(len(table))), int(length),
                                 token_major=kv.layout == "token_major")


def _same_allocator_state(kv, model, cids, mids, what):
    free, ref = kv.pool.export()
    mfree, mref = model.export()
    assert free.tolist() == mfree, f"{what}: free list differs"
    assert ref.tolist() == mref, f"{what}: refcounts differ"
    for c, m in zip(cids, mids):
        tab, ln = kv.pool.get_table(c)
        assert tab.tolist() == model.tables[m] and ln == model.lengths[m], f"{what}: sequence {c}"


def _same_device_metadata(meta, model, mids, p):
    """The padded device table, the lengths and the shared-token counts equal the
    oracle model's tables, lengths and the oracle's shared-prefix counts."""
    table = meta.table.cpu().numpy()
    lens = meta.lens.cpu().numpy()
    want = np.full(table.shape, -1, np.int32)
    for i, m in enumerate(mids):
        t = model.tables[m]
        want[i, :len(t)] = t
    assert np.array_equal(table, want), "device block table"
    assert lens.tolist() == [model.lengths[m] for m in mids], "device lengths"
    if meta.shared is not None:
        sh = meta.shared.cpu().numpy()
        exp = [0] + [olayout.shared_prefix_tokens(model.tables[a], model.lengths[a],
                                                  model.tables[b], model.lengths[b], p)
                     for a, b in zip(mids[:-1], mids[1:])]
        assert sh.tolist() == exp, "device shared-token counts"


def _decode_full_size(cfg):
    import torch
    from paged_kv_cache_399_amd.session import PagedKVCache
    b, hq, hkv, d, p = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    w = make_workload(cfg, 0, "cuda", extra_steps=BENCH_STEPS)
    kv = PagedKVCache(w.num_blocks, p, hkv, d, w.torch_dtype, "cuda", w.free_order,
                      fill=float("nan"))
    model = PoolModel(w.num_blocks, p, w.free_order)
    if cfg.prefix_len:
        root = kv.new_sequences(1)[0]
        mroot = model.seq_create()
        s_pfx = kv.write([root], [cfg.prefix_len], w.prefix_k, w.prefix_v)
        m_pfx, _ = model.append_slots([mroot], [cfg.prefix_len])
        assert s_pfx.tolist() == m_pfx
        seqs = [root] + [kv.fork(root) for _ in range(b - 1)]
        mids = [mroot] + [model.fork(mroot) for _ in range(b - 1)]
    else:
        seqs = kv.new_sequences(b)
        mids = [model.seq_create() for _ in range(b)]
    priv = (w.lengths - cfg.prefix_len).astype(np.int64)
    slots, cow = kv.pool.append_slots(seqs, priv)
    mslots, mcow = model.append_slots(mids, priv.tolist())
    assert len(cow) == len(mcow) == 0
    assert slots.tolist() == mslots, "bulk-append slots"
    _same_allocator_state(kv, model, seqs, mids, "after the bulk append")
    kv.write_slots(torch.from_numpy(slots).cuda(), w.ctx_k, w.ctx_v)
    max_len = int(w.lengths.max()) + BENCH_STEPS
    total = int(w.lengths.sum()) + b * BENCH_STEPS
    meta = kv.prepare(seqs, -(-max_len // p), hq, max_len, total)
    step = kv.append_decode_tokens(meta, w.step_k[0], w.step_v[0])
    mstep, _ = model.append_slots(mids, [1] * b)
    assert step.tolist() == mstep, "decode-step slots"
    _same_allocator_state(kv, model, seqs, mids, "after the decode append")
    out = torch.full_like(w.q, float("nan"))
    kv.attend(meta, w.q, out)
    torch.cuda.synchronize()
    _same_device_metadata(meta, model, mids, p)
    got_all = out.double().cpu().numpy()
    worst = 0.0
    pk, pv = (host_bits(w.prefix_k), host_bits(w.prefix_v)) if cfg.prefix_len else (None, None)
    checked_prefix = False
    for i in range(b):
        k, v = w.seq_kv(i)
        k = torch.cat([k, w.step_k[0, i:i + 1]], 0)
        v = torch.cat([v, w.step_v[0, i:i + 1]], 0)
        kb, vb = host_bits(k), host_bits(v)
        ref = oatt.decode(host_bits(w.q[i]), kb, vb)
        err = float(np.abs(got_all[i] - ref).max())
        assert np.isfinite(got_all[i]).all(), f"sequence {i}: non-finite output"
        assert err <= BF16_TOL, f"sequence {i} (length {len(kb)}): max abs err {err}"
        worst = max(worst, err)
        m = mids[i]
        tab = model.tables[m]
        if cfg.prefix_len:
            # the shared prefix blocks are read back once; each sequence's own blocks always
            own = cfg.prefix_len // p
            if not checked_prefix:
                ck, cv = _cache_rows(kv, tab[:own], cfg.prefix_len)
                assert np.array_equal(ck, pk) and np.array_equal(cv, pv), "shared prefix rows"
                checked_prefix = True
            assert tab[:own] == model.tables[mids[0]][:own]
            ck, cv = _cache_rows(kv, tab[own:], len(kb) - own * p)
            assert np.array_equal(ck, kb[own * p:]) and np.array_equal(cv, vb[own * p:]), \
                f"sequence {i}: cache rows differ"
        else:
            ck, cv = _cache_rows(kv, tab, len(kb))
            assert np.array_equal(ck, kb) and np.array_equal(cv, vb), f"sequence {i}: cache rows differ"
    say(f"  {cfg.name}: {b} of {b} sequences, {int(w.lengths.sum())} context tokens, "
        f"max err {worst:.3e}")


def test_long_decode_full_size_every_sequence():
    _decode_full_size(CONFIGS["long"])


@pytest.mark.parametrize("page", [8, 16, 32])
def test_prefix_decode_full_size_every_sequence(page):
    cfg = CONFIGS["prefix"]
    _decode_full_size(cfg if page == cfg.block_size else cfg.with_block_size(page))


@pytest.mark.parametrize("name", ["prefill", "prefill_chunk"])
def test_prefill_full_size_every_sequence(name):
    import torch
    from paged_kv_cache_399_amd import paged_attention_prefill
    from paged_kv_cache_399_amd.session import PagedKVCache
    cfg = PREFILL_CONFIGS[name]
    b, hq, hkv, d, p = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    w = make_prefill_workload(cfg, 0, "cuda")
    kv = PagedKVCache(w.num_blocks, p, hkv, d, torch.bfloat16, "cuda", w.free_order, fill=float("nan"))
    model = PoolModel(w.num_blocks, p, w.free_order)
    seqs = kv.new_sequences(b)
    mids = [model.seq_create() for _ in range(b)]
    if cfg.context:
        slots, _ = kv.pool.append_slots(seqs, [cfg.context] * b)
        mslots, _ = model.append_slots(mids, [cfg.context] * b)
        assert slots.tolist() == mslots
        kv.write_slots(torch.from_numpy(slots).cuda(), w.ctx_k, w.ctx_v)
    total = cfg.context + cfg.new
    m = kv.prepare(seqs, -(-total // p), hq, total, b * total)
    out = torch.full_like(w.q, float("nan"))
    kv.extend(m, [cfg.new] * b, w.new_k, w.new_v, w.q, out)
    model.append_slots(mids, [cfg.new] * b)
    _same_allocator_state(kv, model, seqs, mids, "after the prefill append")
    # the timed call: attention alone on the final state, into a fresh output
    out2 = torch.full_like(w.q, float("nan"))
    paged_attention_prefill(out2, w.q, kv.k_cache, kv.v_cache, m.table, m.lens, m.query_start, cfg.new)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    _same_device_metadata(m, model, mids, p)
    got_all = out.double().cpu().numpy()
    worst = 0.0
    for i in range(b):
        rows = slice(i * cfg.new, (i + 1) * cfg.new)
        k = torch.cat([w.ctx_k[i * cfg.context:(i + 1) * cfg.context], w.new_k[rows]], 0)
        v = torch.cat([w.ctx_v[i * cfg.context:(i + 1) * cfg.context], w.new_v[rows]], 0)
        kb, vb = host_bits(k), host_bits(v)
        ref = oatt.prefill(host_bits(w.q[rows]), kb, vb)
        err = float(np.abs(got_all[rows] - ref).max())
        assert err <= BF16_TOL, f"sequence {i}: max abs err {err}"
        worst = max(worst, err)
        ck, cv = _cache_rows(kv, model.tables[mids[i]], total)
        assert np.array_equal(ck, kb) and np.array_equal(cv, vb), f"sequence {i}: cache rows differ"
    say(f"  {name}: {b} of {b} sequences, max err {worst:.3e}")
