"""Pins of the float64 attention oracle to things other than itself."""
import math

import numpy as np
import pytest
import torch

from oracle import attention


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
