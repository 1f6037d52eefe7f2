"""Fan-out sharing with real copy-on-write copies, through the library, against the oracle.

Prompts are shared by several sequences ("pagedattention" topic page, fourth
paragraph: parallel samples and beams point at the same blocks and copy on
divergence).  Prompt lengths mostly end inside a block, so the first token
each sharer appends copies the shared partial block.  After every step the
slots, the copy-on-write pairs and the whole K/V caches must equal the oracle
pool model's bit for bit, and every sequence's attention must match float64.
A churn phase frees beams and forks new ones from beams that have diverged.
"""
import dataclasses

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import layout as olayout
from oracle.pool_model import PoolModel
from synth import BEAM_CONFIGS, make_beam_workload
from tests.paged_case import BF16_TOL, F32_REL_TOL, host_bits, say

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


class Mirror:
    """The library's cache next to the oracle's model of it."""

    def __init__(self, w):
        import torch
        from paged_kv_cache_399_amd.session import PagedKVCache
        cfg = w.cfg
        self.cfg, self.w = cfg, w
        self.kv = PagedKVCache(w.num_blocks, cfg.block_size, cfg.num_kv_heads, cfg.head_dim,
                               w.torch_dtype, "cuda", w.free_order, fill=7.0)
        self.model = PoolModel(w.num_blocks, cfg.block_size, w.free_order)
        fill = host_bits(torch.full((1,), 7.0, dtype=w.torch_dtype))[0]
        self.kc = np.full(host_bits(self.kv.k_cache).shape, fill, dtype=fill.dtype)
        self.vc = np.full(host_bits(self.kv.v_cache).shape, fill, dtype=fill.dtype)
        self.ids = {}        # library sequence id -> oracle sequence id
        self.hist = {}       # library sequence id -> (list of k rows, list of v rows)

    def new_prompt(self, k, v):
        s = self.kv.new_sequences(1)[0]
        ms = self.model.seq_create()
        self.ids[s] = ms
        slots = self.kv.write([s], [len(k)], k, v)
        mslots, cow = self.model.append_slots([ms], [len(k)])
        assert slots.tolist() == mslots and not cow
        olayout.write_tokens(self.kc, self.vc, mslots, host_bits(k), host_bits(v))
        self.hist[s] = ([k], [v])
        return s

    def fork(self, parent):
        c = self.kv.fork(parent)
        self.ids[c] = self.model.fork(self.ids[parent])
        self.hist[c] = (list(self.hist[parent][0]), list(self.hist[parent][1]))
        return c

    def free(self, s):
        self.kv.free(s)
        self.model.free_seq(self.ids.pop(s))
        self.hist.pop(s)

    def step(self, meta, k, v):
        """One token for every sequence of the batch, then attention."""
        import torch
        seqs = [int(s) for s in meta.seqs]
        mslots, mcow = self.model.append_slots([self.ids[s] for s in seqs], [1] * len(seqs))
        slots = self.kv.append_decode_tokens(meta, k, v)
        assert slots.tolist() == mslots
        for src, dst in mcow:
            olayout.copy_block(self.kc, self.vc, src, dst)
        olayout.write_tokens(self.kc, self.vc, mslots, host_bits(k), host_bits(v))
        for i, s in enumerate(seqs):
            self.hist[s][0].append(k[i:i + 1])
            self.hist[s][1].append(v[i:i + 1])
        out = torch.full_like(self.w.q[:len(seqs)], float("nan"))
        self.kv.attend(meta, self.w.q[:len(seqs)].contiguous(), out)
        torch.cuda.synchronize()
        return out, len(mcow)

    def check(self, meta, out):
        assert np.array_equal(host_bits(self.kv.k_cache), self.kc)
        assert np.array_equal(host_bits(self.kv.v_cache), self.vc)
        worst = 0.0
        import torch
        for i, s in enumerate(int(x) for x in meta.seqs):
            k = torch.cat(self.hist[s][0], 0)
            v = torch.cat(self.hist[s][1], 0)
            ref = oatt.decode(host_bits(self.w.q[i]), host_bits(k), host_bits(v))
            got = out[i].double().cpu().numpy()
            err = float(np.abs(got - ref).max())
            lim = BF16_TOL if self.cfg.dtype == "bf16" else F32_REL_TOL * max(1.0, float(np.abs(ref).max()))
            assert err <= lim, f"sequence {s}: max abs err {err}"
            worst = max(worst, err)
        return worst


def _prepare(mirror, seqs, extra):
    lens = [mirror.kv.pool.get_table(s)[1] for s in seqs]
    p = mirror.cfg.block_size
    mx = max(lens) + extra
    return mirror.kv.prepare(seqs, -(-mx // p), mirror.cfg.num_q_heads, mx, sum(lens) + extra * len(seqs))


@pytest.mark.parametrize("dtype,hq,hkv,d,p", [
    ("bf16", 16, 4, 128, 16), ("bf16", 8, 8, 64, 8), ("bf16", 32, 8, 128, 32), ("f32", 8, 2, 64, 16),
])
def test_fanout_copy_on_write_and_churn(dtype, hq, hkv, d, p):
    cfg = dataclasses.replace(BEAM_CONFIGS["beam"], name="beam_small", groups=6, fanout=4,
                              num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=p, dtype=dtype,
                              length_lo=1, length_hi=300, pool_headroom=3.0)
    steps = 4
    w = make_beam_workload(cfg, seed=9, device="cuda", steps=steps + 2)
    mir = Mirror(w)
    seqs = []
    for gi in range(cfg.groups):
        lo, hi = int(w.cu[gi]), int(w.cu[gi + 1])
        root = mir.new_prompt(w.prompt_k[lo:hi], w.prompt_v[lo:hi])
        seqs += [root] + [mir.fork(root) for _ in range(cfg.fanout - 1)]
    expected_copies = (cfg.fanout - 1) * int(np.sum(w.prompt_lengths % p != 0))
    meta = _prepare(mir, seqs, steps + 2)
    copies = []
    for s in range(steps):
        out, n_cow = mir.step(meta, w.step_k[s], w.step_v[s])
        copies.append(n_cow)
        err = mir.check(meta, out)
        say(f"  step {s}: {n_cow} block copies, max err {err:.3e}")
    assert copies[0] == expected_copies and sum(copies[1:]) == 0
    # churn: drop beam 1 of every group, fork a new beam from beam 0
    new = []
    for gi in range(cfg.groups):
        grp = seqs[gi * cfg.fanout:(gi + 1) * cfg.fanout]
        mir.free(grp[1])
        grp[1] = mir.fork(grp[0])
        new += grp
    meta = _prepare(mir, new, 2)
    for s in range(steps, steps + 2):
        out, n_cow = mir.step(meta, w.step_k[s], w.step_v[s])
        err = mir.check(meta, out)
        say(f"  churn step {s}: {n_cow} block copies, max err {err:.3e}")
