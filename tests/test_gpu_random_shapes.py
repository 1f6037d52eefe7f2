"""Seeded random decode cases across the shape space, against the float64 oracle.

Each case draws a dtype, a head grouping, head_dim, block size, key layout,
partition length, decode kernel (automatic or forced, among those that take
the shape) and a batch of context lengths, then checks slots and both caches
bit for bit and attention against float64 through the library's whole decode
step, and the same decode split into a plan and a planned call (bit-identical).
The draws are fixed by the case number, so a failure names its case.
"""
import numpy as np
import pytest

from synth import DecodeConfig
from tests.paged_case import build_case, check_attention, expected_caches, host_bits, say

pytestmark = pytest.mark.gpu

N_CASES = 24


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


def _draw(case):
    rng = np.random.default_rng(7000 + case)
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    d = int(rng.choice([64, 128, 64, 128, 32, 96]))
    paths = ["generic"]
    if d in (64, 128):
        if dtype == "bf16":
            paths.append("mfma")
        if g <= 4:
            paths.append("dpp")
    math = str(rng.choice(["auto"] + paths))
    if math == "mfma" or (math == "auto" and dtype == "bf16" and d in (64, 128) and g >= 2):
        p = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    elif math == "dpp" or (math == "auto" and d in (64, 128)):
        epc = 8 if dtype == "bf16" else 4
        p = int(rng.choice([epc, 2 * epc, 4 * epc, 8 * epc]))
    else:
        p = int(rng.choice([1, 2, 3, 5, 8, 16]))
    layout = "token_major" if rng.random() < 0.3 else "head_major"
    part = int(rng.choice([0, 0, 64, 128, 512, 2048]))
    b = int(rng.integers(1, 24))
    lengths = rng.integers(1, int(rng.choice([40, 300, 2500])), size=b).tolist()
    if rng.random() < 0.3:
        lengths[0] = int(rng.integers(3000, 9000))
    return dict(dtype=dtype, hq=hkv * g, hkv=hkv, d=d, p=p, math=math, layout=layout, part=part,
                lengths=lengths)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode_case(monkeypatch, case):
    c = _draw(case)
    say(f"  case {case}: {c['dtype']} Hq={c['hq']} Hkv={c['hkv']} D={c['d']} P={c['p']} "
        f"math={c['math']} layout={c['layout']} part={c['part']} B={len(c['lengths'])} "
        f"max L={max(c['lengths'])}")
    if c["math"] != "auto":
        monkeypatch.setenv("PKV_DECODE_MATH", c["math"])
    if c["part"]:
        monkeypatch.setenv("PKV_PARTITION_TOKENS", str(c["part"]))
    cfg = DecodeConfig(f"random_{case}", len(c["lengths"]), c["hq"], c["hkv"], c["d"], c["p"], c["dtype"],
                       "fixed", fixed_lengths=tuple(c["lengths"]))
    kc_case = build_case(cfg, seed=case, fill=7.0, layout=c["layout"])
    import torch
    fill = host_bits(torch.full((1,), 7.0, dtype=kc_case.w.torch_dtype))[0]
    kc, vc, (pfx, pre, dec) = expected_caches(kc_case, fill)
    assert np.array_equal(kc_case.prefill_slots, pre) and np.array_equal(kc_case.decode_slots, dec)
    view = np.uint32 if kc.dtype == np.float32 else kc.dtype
    assert np.array_equal(np.ascontiguousarray(host_bits(kc_case.kv.k_cache)).view(view), kc.view(view))
    assert np.array_equal(np.ascontiguousarray(host_bits(kc_case.kv.v_cache)).view(view), vc.view(view))
    err = check_attention(kc_case)
    # the same decode split into plan + planned call, on a workspace cleared of
    # the full call's plan: bit-identical
    kv, m = kc_case.kv, kc_case.meta
    m.workspace.zero_()
    kv.plan(m)
    out_p = torch.full_like(kc_case.w.q, float("nan"))
    kv.attend(m, kc_case.w.q, out_p, planned=True)
    torch.cuda.synchronize()
    assert torch.equal(out_p, kc_case.out), "planned decode differs from the full call"
    say(f"  case {case}: max err {err:.3e}")


def _draw_prefill(case):
    rng = np.random.default_rng(9100 + case)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    d = int(rng.choice([64, 128]))
    p = int(rng.choice([8, 16, 32, 64, 128, 256]))
    layout = "token_major" if rng.random() < 0.3 else "head_major"
    b = int(rng.integers(1, 6))
    ctx = rng.integers(0, int(rng.choice([50, 700, 3000])), size=b).tolist()
    new = rng.integers(1, int(rng.choice([20, 150, 400])), size=b).tolist()
    return dict(hq=hkv * g, hkv=hkv, d=d, p=p, layout=layout, ctx=ctx, new=new)


@pytest.mark.parametrize("case", range(16))
def test_random_prefill_case(case):
    from tests.test_gpu_prefill import _run
    from tests.paged_case import BF16_TOL
    c = _draw_prefill(case)
    say(f"  prefill case {case}: Hq={c['hq']} Hkv={c['hkv']} D={c['d']} P={c['p']} "
        f"layout={c['layout']} ctx={c['ctx']} new={c['new']}")
    out, ref, _ = _run(c["hq"], c["hkv"], c["d"], c["p"], c["ctx"], c["new"], seed=case, layout=c["layout"])
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    say(f"  prefill case {case}: max err {err:.3e}")
    assert err <= BF16_TOL
