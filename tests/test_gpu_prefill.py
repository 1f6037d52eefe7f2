"""Paged prefill attention (a chunk of appended tokens attending causally) against float64.

Each sequence first holds a context written through the library, then receives
a chunk of new tokens through PagedKVCache.extend (slots, copy-on-write,
incremental table upload, cache_append, prefill kernel).  Every new token's
output is compared with oracle.attention.prefill over the sequence's keys and
values in logical order (bf16: max |err| <= 2e-2 against float64).
"""
import dataclasses

import numpy as np
import pytest

from oracle import attention as oatt
from tests.paged_case import BF16_TOL, host_bits, say

pytestmark = pytest.mark.gpu


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


def _run(hq, hkv, d, p, ctx_lens, new_lens, seed, free_order=None, fill=None, layout="head_major",
         kscale=None, scale=None):
    """Returns (outputs [tokens, Hq, D] on the host as float64, oracle rows, pool).

    kscale(t, L), if given, multiplies the key of position t of an L-token
    sequence (before rounding to bf16); scale is passed to the kernel and the
    oracle alike (None: 1 / sqrt(D))."""
    import torch
    from paged_kv_cache_399_amd.session import PagedKVCache
    ctx_lens = np.asarray(ctx_lens, np.int64)
    new_lens = np.asarray(new_lens, np.int64)
    b = len(ctx_lens)
    total = ctx_lens + new_lens
    need = int(np.sum(-(-total // p))) + 4
    nb = 2 * need
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32) if free_order is None \
        else free_order
    g = torch.Generator(device="cuda").manual_seed(seed)
    kv_all = []
    for t in total:
        k = torch.randn((int(t), hkv, d), generator=g, device="cuda")
        if kscale is not None:
            pos = torch.arange(int(t), device="cuda", dtype=torch.float32)
            k = k * kscale(pos, float(t))[:, None, None]
        kv_all.append((k.to(torch.bfloat16),
                       torch.randn((int(t), hkv, d), generator=g, device="cuda").to(torch.bfloat16)))
    q = torch.randn((int(new_lens.sum()), hq, d), generator=g, device="cuda").to(torch.bfloat16)
    kv = PagedKVCache(nb, p, hkv, d, torch.bfloat16, "cuda", order,
                      fill=float("nan") if fill is None else fill, layout=layout)
    seqs = kv.new_sequences(b)
    for i, s in enumerate(seqs):
        if ctx_lens[i]:
            kv.write([s], [int(ctx_lens[i])], kv_all[i][0][:ctx_lens[i]], kv_all[i][1][:ctx_lens[i]])
    mb = -(-int(total.max()) // p)
    m = kv.prepare(seqs, mb, hq, int(total.max()), int(total.sum()))
    kn = torch.cat([kv_all[i][0][ctx_lens[i]:] for i in range(b)], 0).contiguous()
    vn = torch.cat([kv_all[i][1][ctx_lens[i]:] for i in range(b)], 0).contiguous()
    out = torch.full_like(q, float("nan"))
    kv.extend(m, new_lens, kn, vn, q, out, scale=scale)
    kv._last_q = q
    kv._last_k = [k for k, _ in kv_all]
    torch.cuda.synchronize()
    refs = []
    row = 0
    for i in range(b):
        n = int(new_lens[i])
        refs.append(oatt.prefill(host_bits(q[row:row + n]), host_bits(kv_all[i][0]),
                                 host_bits(kv_all[i][1]), scale))
        row += n
    return out, np.concatenate(refs, 0) if refs else np.zeros((0, hq, d)), kv


@pytest.mark.parametrize("hq,hkv,d,p", [
    (8, 8, 128, 16), (8, 4, 64, 8), (16, 4, 128, 16), (32, 8, 128, 32), (16, 2, 64, 16),
    (16, 1, 128, 16),
    # head groups that are not powers of two: G = 3, 5, 6, 7, 12, 10 (one, one, two, one,
    # four and two heads per workgroup)
    (3, 1, 128, 16), (10, 2, 64, 8), (12, 2, 128, 16), (28, 4, 128, 16), (24, 2, 128, 32),
    (40, 4, 64, 16),
    # more than 16 query heads per KV head (the session's decode sizing takes them too)
    (32, 1, 128, 16), (48, 2, 64, 8),
])
def test_prefill_chunks_match_oracle(hq, hkv, d, p):
    ctx = [0, 0, 5, 100, 333, 16, 1000]
    new = [1, 77, 16, 17, 64, 100, 150]
    out, ref, _ = _run(hq, hkv, d, p, ctx, new, seed=hq + d + p)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    say(f"  max err {err:.3e}")
    assert err <= BF16_TOL


def test_fresh_prompts_are_full_causal_prefill():
    out, ref, _ = _run(32, 8, 128, 16, [0, 0, 0], [1, 255, 700], seed=3)
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    say(f"  max err {err:.3e}")
    assert err <= BF16_TOL


def test_prefill_block_permutation_is_bit_identical_and_poison_free():
    import torch
    ctx, new = [40, 0, 300], [30, 90, 33]
    a, _, kva = _run(16, 4, 128, 16, ctx, new, seed=11)
    nb = kva.num_blocks
    other = np.random.default_rng(5).permutation(nb).astype(np.int32)
    b, _, _ = _run(16, 4, 128, 16, ctx, new, seed=11, free_order=other)
    c, _, _ = _run(16, 4, 128, 16, ctx, new, seed=11, fill=0.0)
    assert torch.equal(a, b)
    assert torch.equal(a, c)


@pytest.mark.parametrize("p", [64, 128, 256])
def test_large_blocks(p):
    """Blocks of 64-256 tokens: several 16-key staging groups and several
    64-key chunks per block, a last block filled only in part, and contexts
    that end inside a block."""
    ctx = [0, 5, 300, 1000]
    new = [150, 77, 64, 200]
    out, ref, _ = _run(16, 4, 128, p, ctx, new, seed=p)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    say(f"  p={p}: max err {err:.3e}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("p", [8, 16, 32])
@pytest.mark.parametrize("shape", ["rising", "falling"])
def test_running_reference_moves_within_a_sequence(shape, p):
    """Large scores: keys that grow (or shrink) 8-fold along the sequence, at
    twice the default scale (scores up to about 70 in log2 units).  Rising,
    later 64-key chunks beat the first chunk's maximum by far more than 2^8 in
    probability, so each query's running reference moves several times and
    the accumulators are rescaled; falling, the early keys dominate.  Outputs
    stay within the bf16 bound: at these magnitudes a score rounded through
    bf16 anywhere on the way (a pre-scaled query, say) is off by ~0.1."""
    import torch
    if shape == "rising":
        ramp = lambda t, n: 1.0 + 7.0 * t / n  # noqa: E731
    else:
        ramp = lambda t, n: 8.0 - 7.0 * t / n  # noqa: E731
    scale = 2.0 / np.sqrt(128)
    ctx, new = [0, 600, 1500], [300, 200, 130]
    out, ref, kv = _run(16, 4, 128, p, ctx, new, seed=21 + p, kscale=ramp, scale=scale)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    # the data does what the test is for (rising): for the last query of the
    # longest sequence, some chunk's maximum score (log2 units) passes the
    # first chunk's by more than 8
    q = oatt.as_f64(host_bits(kv._last_q[-1]))      # [Hq, D]: sees every key of sequence 2
    keys = oatt.as_f64(host_bits(kv._last_k[2]))    # [L, Hkv, D]
    s2 = np.einsum("hd,lhd->lh", q[::4], keys) * scale * np.log2(np.e)  # one query head per KV head
    chunk_max = np.array([s2[c:c + 64].max() for c in range(0, len(s2), 64)])
    moves = int(np.sum(np.maximum.accumulate(chunk_max)[1:] > chunk_max[0] + 8))
    say(f"  {shape} p={p}: max err {err:.3e}, chunks past the first chunk's maximum + 8: {moves}")
    if shape == "rising":
        assert moves > 0
    assert err <= BF16_TOL


@pytest.mark.parametrize("hq,hkv,d,p", [(16, 4, 128, 16), (8, 8, 64, 8), (32, 8, 128, 32)])
def test_token_major_key_layout(hq, hkv, d, p):
    """Keys stored [blocks, P, Hkv, D]: same outputs as the oracle, and bit for
    bit the same as the head-major cache on the same inputs."""
    import torch
    ctx, new = [0, 5, 100, 333], [77, 16, 17, 64]
    out, ref, _ = _run(hq, hkv, d, p, ctx, new, seed=p + d, layout="token_major")
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    say(f"  max err {err:.3e}")
    assert err <= BF16_TOL
    head, _, _ = _run(hq, hkv, d, p, ctx, new, seed=p + d)
    assert torch.equal(out, head)


@pytest.mark.parametrize("p", [8, 16])
def test_contexts_longer_than_the_table_window(p):
    """Contexts past 1024 blocks make the kernel move its block-table window
    (every 1024 blocks) while it walks the keys."""
    ctx = [9000, 300, 17000 if p == 16 else 8190]
    new = [40, 77, 33]
    out, ref, _ = _run(16, 4, 128, p, ctx, new, seed=p + 1)
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    say(f"  p={p}: max err {err:.3e}")
    assert err <= BF16_TOL


def test_max_query_len_below_the_new_tokens_flags_and_leaves_rows_unwritten():
    """The grid covers ceil(max_query_len / BT) tiles of BT query tokens per
    sequence; a sequence with more new tokens keeps its later rows unwritten
    and flags PKV_DEVERR_CONTEXT_LEN (0x8).  Rows the grid covers are the
    full call's rows bit for bit."""
    import torch
    import paged_kv_cache_399_amd as pkv
    from paged_kv_cache_399_amd import paged_attention_prefill
    hq, hkv, d, p = 32, 8, 128, 16
    new = [100, 30]
    out, ref, kv = _run(hq, hkv, d, p, [50, 20], new, seed=6)
    assert float(np.abs(out.double().cpu().numpy() - ref).max()) <= BF16_TOL
    m = kv._meta
    bt = 16 * (8 // min(hq // hkv, 8))           # query tokens per workgroup tile
    short = 40
    covered = -(-short // bt) * bt
    assert new[0] > covered >= new[1]
    q = kv._last_q
    out2 = torch.full_like(out, float("nan"))
    paged_attention_prefill(out2, q, kv.k_cache, kv.v_cache, m.table, m.lens, m.query_start, short)
    with pytest.raises(pkv.PkvError) as e:
        pkv.check_device_errors()
    assert "0x8" in str(e.value)
    assert torch.equal(out2[:covered], out[:covered])
    assert torch.isnan(out2[covered:new[0]].float()).all()
    assert torch.equal(out2[new[0]:], out[new[0]:])
