"""Pins of the float64 attention oracle to things other than itself."""
import math

import numpy as np
import pytest
import torch

from oracle import attention
from oracle import attention as oatt


def _rand(rng, *shape):
    return rng.uniform(-1, 1, size=shape)


def test_bf16_patterns_are_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x0000, 0x8000], np.uint16)
    got = attention.bf16_bits_to_f64(bits)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, 0.0, -0.0]
    assert got.tolist() == want
    # and agrees with torch's own bf16 -> float64 conversion on random patterns
    r = np.random.default_rng(0).integers(0, 0x7F80, size=4096, dtype=np.uint16)
    t = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(attention.bf16_bits_to_f64(r), t)


@pytest.mark.parametrize("hq,hkv,length,d", [(1, 1, 1, 8), (1, 1, 4, 8), (4, 2, 5, 3),
                                             (6, 3, 7, 4), (2, 1, 9, 5)])
def test_numpy_matches_brute_force(hq, hkv, length, d):
    rng = np.random.default_rng(hq * 100 + length)
    q, k, v = _rand(rng, hq, d), _rand(rng, length, hkv, d), _rand(rng, length, hkv, d)
    got = attention.decode(q, k, v)
    want = np.array(attention.decode_brute(q, k, v))
    assert np.abs(got - want).max() < 1e-13


@pytest.mark.parametrize("hq,hkv,length,d", [(8, 8, 33, 64), (32, 8, 100, 128), (4, 1, 17, 16)])
def test_matches_torch_sdpa_float64(hq, hkv, length, d):
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((hq, d)), rng.standard_normal((length, hkv, d)), \
        rng.standard_normal((length, hkv, d))
    g = hq // hkv
    qt = torch.from_numpy(q)[None, :, None, :]                              # [1,Hq,1,D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)[None]  # [1,Hq,L,D]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0, :].numpy()
    assert np.abs(attention.decode(q, k, v) - ref).max() < 1e-12


def test_two_token_closed_form():
    """Scores x and 0 give weights e^x / (1 + e^x) and 1 / (1 + e^x)."""
    d = 16
    q = np.zeros((1, d)); q[0, 0] = 2.0
    k = np.zeros((2, 1, d)); k[0, 0, 0] = 3.0            # scaled score 6 / sqrt(16) = 1.5
    v = np.zeros((2, 1, d)); v[0, 0, 1] = 1.0; v[1, 0, 2] = 1.0
    out = attention.decode(q, k, v)
    x = 6.0 / math.sqrt(d)
    assert out[0, 1] == pytest.approx(math.exp(x) / (1 + math.exp(x)), abs=1e-15)
    assert out[0, 2] == pytest.approx(1 / (1 + math.exp(x)), abs=1e-15)
    assert out[0, 0] == 0.0


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 4, 8), _rand(rng, 1, 2, 8), _rand(rng, 1, 2, 8)
    out = attention.decode(q, k, v)
    assert np.array_equal(out, np.repeat(v[0], 2, axis=0))


def test_zero_query_or_equal_keys_give_the_mean_value():
    rng = np.random.default_rng(2)
    v = _rand(rng, 11, 1, 8)
    k = _rand(rng, 11, 1, 8)
    out = attention.decode(np.zeros((1, 8)), k, v)
    assert np.abs(out[0] - v[:, 0].mean(0)).max() < 1e-15
    keq = np.repeat(k[:1], 11, axis=0)
    out = attention.decode(_rand(rng, 1, 8), keq, v)
    assert np.abs(out[0] - v[:, 0].mean(0)).max() < 1e-15


def test_empty_sequence_gives_zeros():
    out = attention.decode(np.ones((2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)))
    assert np.array_equal(out, np.zeros((2, 4)))


def test_grouped_heads_equal_repeated_kv_heads():
    rng = np.random.default_rng(4)
    hq, hkv, length, d = 8, 2, 13, 8
    q, k, v = _rand(rng, hq, d), _rand(rng, length, hkv, d), _rand(rng, length, hkv, d)
    g = hq // hkv
    mha = attention.decode(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1))
    assert np.abs(attention.decode(q, k, v) - mha).max() < 1e-15


def test_grouping_is_contiguous():
    """Query head h reads KV head h // G: changing KV head 1 moves heads 2..3 only."""
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 4, 4), _rand(rng, 6, 2, 4), _rand(rng, 6, 2, 4)
    a = attention.decode(q, k, v)
    v2 = v.copy(); v2[:, 1] += 1.0
    b = attention.decode(q, k, v2)
    assert np.array_equal(a[:2], b[:2]) and not np.allclose(a[2:], b[2:])


@pytest.mark.parametrize("t", [1, 3, 16, 32, 100])
def test_partitioned_merge_equals_direct(t):
    rng = np.random.default_rng(t)
    q, k, v = rng.standard_normal((8, 16)) * 3, rng.standard_normal((77, 2, 16)), \
        rng.standard_normal((77, 2, 16))
    assert np.abs(attention.partitioned(q, k, v, t) - attention.decode(q, k, v)).max() < 1e-13


def test_bf16_inputs_convert_before_the_maths():
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((9, 1, 8)).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    q = bits[0]
    out = attention.decode(q, bits, bits)
    ref = attention.decode(x[0].to(torch.float64).numpy(), x.to(torch.float64).numpy(),
                           x.to(torch.float64).numpy())
    assert np.array_equal(out, ref)


def _prefill_brute(q, k, v):
    """Pure-Python causal attention of the last n tokens (positions L - n ..)."""
    q, k, v = oatt.as_f64(q).tolist(), oatt.as_f64(k).tolist(), oatt.as_f64(v).tolist()
    n, hq, d = len(q), len(q[0]), len(q[0][0])
    l, hkv = len(k), len(k[0])
    g = hq // hkv
    scale = 1.0 / math.sqrt(d)
    out = []
    for i in range(n):
        last = l - n + i
        row = []
        for h in range(hq):
            kv = h // g
            sc = [scale * sum(q[i][h][x] * k[t][kv][x] for x in range(d)) for t in range(last + 1)]
            top = max(sc)
            w = [math.exp(s - top) for s in sc]
            tot = sum(w)
            row.append([sum(w[t] * v[t][kv][x] for t in range(last + 1)) / tot for x in range(d)])
        out.append(row)
    return out


@pytest.mark.parametrize("hq,hkv,l,n,d", [(2, 1, 5, 5, 4), (4, 2, 7, 3, 8), (3, 3, 6, 1, 4)])
def test_prefill_matches_brute_force(hq, hkv, l, n, d):
    rng = np.random.default_rng(l * 10 + n)
    q = rng.uniform(-1, 1, (n, hq, d))
    k = rng.uniform(-1, 1, (l, hkv, d))
    v = rng.uniform(-1, 1, (l, hkv, d))
    assert np.allclose(oatt.prefill(q, k, v), np.array(_prefill_brute(q, k, v)), rtol=0, atol=1e-13)


@pytest.mark.parametrize("hq,hkv,l,n", [(8, 2, 40, 40), (4, 4, 33, 9), (6, 1, 17, 16)])
def test_prefill_matches_torch_sdpa_with_causal_mask(hq, hkv, l, n):
    import torch
    rng = np.random.default_rng(hq + l)
    d = 16
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((l, hkv, d))
    v = rng.standard_normal((l, hkv, d))
    g = hq // hkv
    kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)      # [Hq, L, D]
    vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
    qt = torch.from_numpy(q).permute(1, 0, 2)                           # [Hq, n, D]
    mask = torch.arange(l)[None, :] <= (l - n + torch.arange(n))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    assert np.allclose(oatt.prefill(q, k, v), ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_prefill_rows_are_decodes_over_the_visible_keys():
    rng = np.random.default_rng(3)
    l, n, hq, hkv, d = 30, 12, 8, 2, 8
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((l, hkv, d))
    v = rng.standard_normal((l, hkv, d))
    out = oatt.prefill(q, k, v)
    for i in range(n):
        last = l - n + i
        assert np.allclose(out[i], oatt.decode(q[i], k[:last + 1], v[:last + 1]), rtol=0, atol=1e-13)
    # the first token of a fresh sequence sees only itself: its value, exactly
    first = oatt.prefill(q[:1], k[:1], v[:1])
    assert np.array_equal(first[0], np.repeat(v[0], hq // hkv, axis=0))
