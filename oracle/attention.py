"""Decode-step attention in float64 over keys and values in logical order.

The pages say only that attention follows each sequence's block table to reach
the right keys and values ("PagedAttention Internals", "The Block Table Map";
"pagedattention" topic page, third paragraph).  What it then computes is the
ordinary scaled dot-product attention of one new query per head:

    out[h] = sum_t softmax_t(scale * <q[h], K[t, g(h)]>) * V[t, g(h)],
    scale = 1 / sqrt(D),  g(h) = h // (Hq / Hkv)   (grouped heads share K/V),

taken over the sequence's tokens t = 0 .. L-1 in logical order.  Here the
keys and values come straight from the generated per-sequence arrays, never
from a paged cache, so the paging under test cannot leak into the reference.
A sequence with L = 0 has no keys; its output is defined as zeros.

``partitioned`` states the split-context identity: attention over a sequence
cut into consecutive partitions equals the merge of per-partition results
(m_p = max score, l_p = sum of exp(score - m_p), o_p = normalised output),
weighting partition p by l_p * exp(m_p - M) with M the overall maximum.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the pattern is the top half of a float32."""
    b = np.asarray(bits)
    assert b.dtype == np.uint16
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """float32 arrays or uint16 bf16 patterns, converted exactly to float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported dtype {x.dtype}")


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float = None) -> np.ndarray:
    """One sequence: q [Hq, D], k / v [L, Hkv, D] -> out [Hq, D], all float64.

    Per KV head g: scores [L, G] = K_g [L, D] . Q_g^T [D, G]; softmax over L
    after subtracting the column maximum (shift invariance keeps it exact);
    out_g [G, D] = W^T [G, L] . V_g [L, D] / column sums.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    hq, d = q.shape
    l, hkv, d2 = k.shape
    assert d2 == d and v.shape == k.shape and hq % hkv == 0
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((hq, d), dtype=np.float64)
    if l == 0:
        return out
    g = hq // hkv
    for j in range(hkv):
        qg = q[j * g:(j + 1) * g]                 # [G, D]
        s = (k[:, j, :] @ qg.T) * scale           # [L, G]
        s -= s.max(axis=0, keepdims=True)
        w = np.exp(s)
        out[j * g:(j + 1) * g] = (w.T @ v[:, j, :]) / w.sum(axis=0)[:, None]
    return out


def decode_brute(q, k, v, scale: float = None) -> List[List[float]]:
    """Pure-Python loops over the same definition, for tiny inputs."""
    q, k, v = as_f64(q).tolist(), as_f64(k).tolist(), as_f64(v).tolist()
    hq, d = len(q), len(q[0])
    l = len(k)
    hkv = len(k[0]) if l else 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    g = hq // hkv
    out = []
    for h in range(hq):
        if l == 0:
            out.append([0.0] * d)
            continue
        kv = h // g
        scores = [scale * sum(q[h][i] * k[t][kv][i] for i in range(d)) for t in range(l)]
        top = max(scores)
        w = [math.exp(s - top) for s in scores]
        tot = sum(w)
        out.append([sum(w[t] * v[t][kv][i] for t in range(l)) / tot for i in range(d)])
    return out


def partition_stats(q, k, v, scale: float = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(m [Hq], l [Hq], o [Hq, D]) of one non-empty partition, float64."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    hq, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = default_scale(d)
    g = hq // hkv
    m = np.empty(hq)
    lsum = np.empty(hq)
    o = np.empty((hq, d))
    for h in range(hq):
        s = (k[:, h // g, :] @ q[h]) * scale
        m[h] = s.max()
        w = np.exp(s - m[h])
        lsum[h] = w.sum()
        o[h] = (w @ v[:, h // g, :]) / lsum[h]
    return m, lsum, o


def merge(parts: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """Combine per-partition (m, l, o) into the attention output."""
    ms = np.stack([p[0] for p in parts])          # [n, Hq]
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[2] for p in parts])         # [n, Hq, D]
    top = ms.max(axis=0)
    w = ls * np.exp(ms - top)                     # [n, Hq]
    return (w[:, :, None] * os_).sum(axis=0) / w.sum(axis=0)[:, None]


def partitioned(q, k, v, part_tokens: int, scale: float = None) -> np.ndarray:
    """Attention computed partition by partition and merged."""
    k, v = as_f64(k), as_f64(v)
    q = as_f64(q)
    l = k.shape[0]
    if l == 0:
        return np.zeros(q.shape)
    parts = [partition_stats(q, k[s:s + part_tokens], v[s:s + part_tokens], scale)
             for s in range(0, l, part_tokens)]
    return merge(parts)


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float = None) -> np.ndarray:
    """Causal attention of a sequence's newest tokens, float64.

    q [n, Hq, D] are the queries of the last n of the sequence's L tokens
    (positions L - n .. L - 1); k / v [L, Hkv, D] are all L tokens in logical
    order.  Query i sees keys 0 .. L - n + i: the tokens before it and itself,
    which is what appending a chunk of tokens to a paged sequence and attending
    from each of them computes.  Per KV head: scores [n, L], masked above the
    causal boundary, softmax per row after subtracting the row maximum, times V.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    n, hq, d = q.shape
    l, hkv, d2 = k.shape
    assert d2 == d and v.shape == k.shape and hq % hkv == 0 and n <= l
    if scale is None:
        scale = default_scale(d)
    g = hq // hkv
    out = np.zeros((n, hq, d), dtype=np.float64)
    pos = (l - n) + np.arange(n)                          # absolute position of each query
    visible = np.arange(l)[None, :] <= pos[:, None]       # [n, L]
    for h in range(hq):
        j = h // g
        s = (q[:, h, :] @ k[:, j, :].T) * scale           # [n, L]
        s = np.where(visible, s, -np.inf)
        s -= s.max(axis=1, keepdims=True)
        w = np.exp(s)
        out[:, h, :] = (w @ v[:, j, :]) / w.sum(axis=1, keepdims=True)
    return out
