"""The decode split into one plan and several planned calls (one per layer).

decode_plan runs the plan kernel alone; paged_attention_decode_planned runs
the partition and merge kernels on that plan.  For every kernel family (DPP,
generic fp32, matrix cores with and without packs, split partitions) the
planned calls over several query tensors ("layers") on one plan must equal
the full decode call on the same state bit for bit, after each decode step's
re-plan, and the full decode must match float64.  A planned call whose
workspace holds a plan for other sizing, or none, computes nothing and sets
the plan error bit.
"""
import numpy as np
import pytest

from synth import CONFIGS
from tests.paged_case import build_case, check_attention, say

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


def _with_headroom(case, steps):
    """A fresh batch description of the case's sequences, sized for `steps`
    more decode tokens per sequence (prepare() fixes the sizing)."""
    kv, w = case.kv, case.w
    p, b = case.cfg.block_size, case.cfg.batch
    max_len = int(w.lengths.max()) + steps
    return kv.prepare(case.seqs, -(-max_len // p), case.cfg.num_q_heads, max_len,
                      int(w.lengths.sum()) + b * steps)


def _q_like(q, rng):
    import torch
    return torch.from_numpy(rng.standard_normal(tuple(q.shape)).astype(np.float32)).to(q.dtype).to(q.device)


@pytest.mark.parametrize("name,forced_t,math", [
    ("tiny", None, None),          # fp32: generic kernel
    ("small_mha", None, None),     # multi-head bf16: matrix cores
    ("small_mha", None, "dpp"),    # the DPP kernel
    ("gqa", None, None), ("gqa", 128, None), ("prefix", None, None), ("prefix", 256, None)])
def test_planned_layers_equal_the_full_decode(monkeypatch, name, forced_t, math):
    import torch
    if forced_t:
        monkeypatch.setenv("PKV_PARTITION_TOKENS", str(forced_t))
    if math:
        monkeypatch.setenv("PKV_DECODE_MATH", math)
    case = build_case(CONFIGS[name], seed=3)
    worst = check_attention(case)
    kv, w = case.kv, case.w
    m = _with_headroom(case, 2)
    zeros = w.q.new_zeros((w.q.shape[0], kv.num_kv_heads, kv.head_dim))
    rng = np.random.default_rng(11)
    layers = 3
    for step in range(2):
        # a decode step: one token per sequence, new lengths, a new plan
        kv.append_decode_tokens(m, zeros, zeros)
        qs = [_q_like(w.q, rng) for _ in range(layers)]
        kv.plan(m)
        planned = []
        for q in qs:                       # every layer on the one plan
            o = torch.full_like(q, float("nan"))
            kv.attend(m, q, o, planned=True)
            planned.append(o)
        for i, q in enumerate(qs):         # the full call re-plans the same lengths
            o = torch.full_like(q, float("nan"))
            kv.attend(m, q, o)
            torch.cuda.synchronize()
            assert torch.equal(planned[i], o), f"step {step}, layer {i}: planned decode differs"
    say(f"  {name} T={forced_t} math={math}: {layers} layers x 2 steps bit-identical; max err {worst:.3e}")
    kv.close()


def test_planned_decode_refuses_another_plan(monkeypatch):
    import torch
    import paged_kv_cache_399_amd as pkv
    case = build_case(CONFIGS["gqa"], seed=5)
    kv, m, w = case.kv, case.meta, case.w
    kv.plan(m)
    # a longer partition (fewer units: the workspace still fits) changes the sizing
    monkeypatch.setenv("PKV_PARTITION_TOKENS", "2048")
    out = torch.full_like(w.q, float("nan"))
    kv.attend(m, w.q, out, planned=True)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a planned decode on another plan wrote output"
    with pytest.raises(pkv.PkvError) as e:
        pkv.check_device_errors()
    assert "(flags 0x20)" in str(e.value)
    monkeypatch.delenv("PKV_PARTITION_TOKENS")
    # a workspace that holds no plan at all
    m.workspace.zero_()
    kv.attend(m, w.q, out, planned=True)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a planned decode without a plan wrote output"
    with pytest.raises(pkv.PkvError) as e:
        pkv.check_device_errors()
    assert "(flags 0x20)" in str(e.value)
    # planning again makes the planned call whole
    kv.plan(m)
    kv.attend(m, w.q, out, planned=True)
    ref = torch.full_like(w.q, float("nan"))
    kv.attend(m, w.q, ref)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    kv.close()


def test_graph_of_planned_layers_replays_like_eager():
    """Capture plan + two planned layers in one graph; replays between eager
    decode steps equal the eager calls on the same state."""
    import torch
    case = build_case(CONFIGS["gqa"], seed=7)
    kv, w = case.kv, case.w
    m = _with_headroom(case, 3)
    kv.upload(m)
    rng = np.random.default_rng(8)
    q1, q2 = _q_like(w.q, rng), _q_like(w.q, rng)
    g1, g2 = torch.full_like(q1, float("nan")), torch.full_like(q2, float("nan"))
    e1, e2 = torch.full_like(q1, float("nan")), torch.full_like(q2, float("nan"))
    kv.plan(m)
    kv.attend(m, q1, g1, planned=True)   # one-time host set-up outside the capture
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s = torch.cuda.current_stream()
        kv.plan(m, stream=s)
        kv.attend(m, q1, g1, stream=s, planned=True)
        kv.attend(m, q2, g2, stream=s, planned=True)
    zeros = w.q.new_zeros((w.q.shape[0], kv.num_kv_heads, kv.head_dim))
    for step in range(3):
        kv.append_decode_tokens(m, zeros, zeros)
        kv.attend(m, q1, e1)
        kv.attend(m, q2, e2)
        kv.check_graph_sizing(m)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g1, e1) and torch.equal(g2, e2), f"replay {step} differs"
    kv.close()
