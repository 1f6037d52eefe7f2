"""Seeded synthetic inputs for paged decode attention.

This module draws random numbers and nothing else: context lengths, the order
in which a pool hands out its free blocks, and the query / key / value tensors.
It holds none of the paged-cache arithmetic (no slot maths, no block tables,
no attention), so that the CPU oracle and the GPU path can both consume the
same inputs without sharing any method code.

The five workloads mirror the decode shapes this library is measured on:

* ``tiny``        3 sequences of lengths [1, 4, 2], page size 2, 16 physical
                  blocks, one head, head_dim 8, fp32 uniform[-1, 1].  These are
                  the lengths of the worked fragmentation example in the
                  "inference-acceleration-pagedattention-vllm" chapter.
* ``small_mha``   batch 8, 8 query heads = 8 KV heads, head_dim 64, block 16,
                  lengths uniform in [1, 512], bf16 N(0, 1), 1024-block pool.
* ``gqa``         batch 64, 32 query / 8 KV heads, head_dim 128, block 16,
                  lengths uniform in [128, 4096], pool 1.25x the blocks needed.
* ``long``        batch 256, 64 query / 8 KV heads, head_dim 128, block 16,
                  lengths log-uniform in [16, 32768], pool 1.25x needed.
* ``prefix``      128 sequences sharing a 2048-token prefix plus private
                  suffixes uniform in [1, 1024], 32 / 8 heads, head_dim 128,
                  block size 8, 16 or 32.

Conventions shared by every consumer:

* ``lengths[b]`` is sequence b's context length at the decode step, counting
  the token that the step itself appends.  Set-up therefore writes
  ``lengths[b] - 1`` tokens and the step writes one more.
* Keys and values are handed out per sequence in logical token order.  For the
  ``prefix`` workload the first ``prefix_len`` tokens of every sequence are the
  same shared arrays.
* bf16 values are float32 draws rounded to bf16 by ``torch.Tensor.to``
  (round to nearest even).  Host consumers read their raw 16-bit patterns.
* Every stream (lengths, pool order, q, k, v, per-step tokens) has its own
  seed derived from ``(seed, stream name)``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "DecodeConfig", "CONFIGS", "stream_seed", "context_lengths", "pool_size",
    "free_order", "Workload", "make_workload", "bf16_bits", "to_numpy_f32",
    "BeamConfig", "BEAM_CONFIGS", "BeamWorkload", "make_beam_workload",
    "PrefillConfig", "PREFILL_CONFIGS", "PrefillWorkload", "make_prefill_workload",
]


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f32" or "bf16"
    length_rule: str                # "fixed", "uniform", "loguniform", "prefix"
    length_lo: int = 0
    length_hi: int = 0
    fixed_lengths: Tuple[int, ...] = ()
    prefix_len: int = 0
    pool_blocks: Optional[int] = None   # explicit pool size; None = 1.25x needed
    pool_headroom: float = 1.25
    value_dist: str = "normal"      # "normal" N(0,1) or "uniform" U[-1,1]

    def with_block_size(self, p: int) -> "DecodeConfig":
        return dataclasses.replace(self, block_size=p, name=f"{self.name}_p{p}")


CONFIGS: Dict[str, DecodeConfig] = {
    "tiny": DecodeConfig("tiny", 3, 1, 1, 8, 2, "f32", "fixed",
                         fixed_lengths=(1, 4, 2), pool_blocks=16,
                         value_dist="uniform"),
    "small_mha": DecodeConfig("small_mha", 8, 8, 8, 64, 16, "bf16", "uniform",
                              length_lo=1, length_hi=512, pool_blocks=1024),
    "gqa": DecodeConfig("gqa", 64, 32, 8, 128, 16, "bf16", "uniform",
                        length_lo=128, length_hi=4096),
    "long": DecodeConfig("long", 256, 64, 8, 128, 16, "bf16", "loguniform",
                         length_lo=16, length_hi=32768),
    "prefix": DecodeConfig("prefix", 128, 32, 8, 128, 16, "bf16", "prefix",
                           length_lo=1, length_hi=1024, prefix_len=2048),
    # multi-head attention (no head sharing) at the GQA workload's lengths: 64
    # sequences, 32 query and 32 KV heads of 128 dims
    "mha": DecodeConfig("mha", 64, 32, 32, 128, 16, "bf16", "uniform",
                        length_lo=128, length_hi=4096),
}


def stream_seed(seed: int, stream: str) -> int:
    """A 63-bit seed for one named random stream of a run seeded with ``seed``."""
    h = hashlib.sha256(f"{int(seed)}/{stream}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _rng(seed: int, stream: str) -> np.random.Generator:
    return np.random.default_rng(stream_seed(seed, stream))


def context_lengths(cfg: DecodeConfig, seed: int) -> np.ndarray:
    """Context length of each sequence at the decode step (int64[B])."""
    rng = _rng(seed, "lengths")
    b = cfg.batch
    if cfg.length_rule == "fixed":
        out = np.asarray(cfg.fixed_lengths, dtype=np.int64)
        assert out.shape == (b,)
        return out
    if cfg.length_rule == "uniform":
        return rng.integers(cfg.length_lo, cfg.length_hi + 1, size=b, dtype=np.int64)
    if cfg.length_rule == "loguniform":
        lo, hi = math.log(cfg.length_lo), math.log(cfg.length_hi + 1)
        out = np.floor(np.exp(rng.uniform(lo, hi, size=b))).astype(np.int64)
        return np.clip(out, cfg.length_lo, cfg.length_hi)
    if cfg.length_rule == "prefix":
        suffix = rng.integers(cfg.length_lo, cfg.length_hi + 1, size=b, dtype=np.int64)
        return cfg.prefix_len + suffix
    raise ValueError(cfg.length_rule)


def _pages(n: int, p: int) -> int:
    return -(-int(n) // int(p))


def pool_size(cfg: DecodeConfig, lengths: np.ndarray, extra_tokens: int = 0) -> int:
    """Number of physical blocks in the pool.

    Sizing only: the explicit size if the workload fixes one, else
    ``pool_headroom`` times the blocks the run can touch (a shared prefix is
    counted once, plus ``extra_tokens`` more tokens per sequence).
    """
    if cfg.pool_blocks is not None:
        return int(cfg.pool_blocks)
    p = cfg.block_size
    need = _pages(cfg.prefix_len, p)
    # a prefix that ends inside a block gives every sharer one private copy
    cow = 1 if cfg.prefix_len % p else 0
    for l in lengths:
        need += _pages(int(l) - cfg.prefix_len + extra_tokens, p) + cow
    return int(math.ceil(cfg.pool_headroom * need))


def free_order(num_blocks: int, seed: int) -> np.ndarray:
    """Seeded permutation of 0..num_blocks-1: the pool's initial free order."""
    return _rng(seed, "pool").permutation(num_blocks).astype(np.int32)


def bf16_bits(t) -> np.ndarray:
    """Raw 16-bit patterns (uint16) of a torch bfloat16 tensor, on the host."""
    import torch
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_numpy_f32(t) -> np.ndarray:
    import torch
    assert t.dtype == torch.float32
    return t.detach().contiguous().cpu().numpy()


@dataclasses.dataclass
class Workload:
    """One decode batch: lengths, pool order and the tensors, in logical order."""
    cfg: DecodeConfig
    seed: int
    lengths: np.ndarray           # int64[B], includes the decode token
    num_blocks: int
    free_order: np.ndarray        # int32[num_blocks]
    q: object                     # torch [B, Hq, D]
    prefix_k: object              # torch [prefix_len, Hkv, D]
    prefix_v: object
    ctx_k: object                 # torch [sum(lengths - prefix_len), Hkv, D]
    ctx_v: object
    cu: np.ndarray                # int64[B+1] offsets of each sequence in ctx_*
    step_k: object                # torch [extra_steps, B, Hkv, D] (bench steps)
    step_v: object

    @property
    def torch_dtype(self):
        import torch
        return torch.float32 if self.cfg.dtype == "f32" else torch.bfloat16

    def seq_kv(self, b: int):
        """(k, v) of sequence b in logical order, as torch tensors on their device."""
        import torch
        lo, hi = int(self.cu[b]), int(self.cu[b + 1])
        k, v = self.ctx_k[lo:hi], self.ctx_v[lo:hi]
        if self.cfg.prefix_len:
            k = torch.cat([self.prefix_k, k], 0)
            v = torch.cat([self.prefix_v, v], 0)
        return k, v


def _draw(cfg: DecodeConfig, shape, seed: int, stream: str, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, stream))
    if cfg.value_dist == "uniform":
        x = torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0
    else:
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if cfg.dtype == "bf16":
        x = x.to(torch.bfloat16)
    return x


def make_workload(cfg: DecodeConfig, seed: int = 0, device="cpu",
                  extra_steps: int = 0, lengths: Optional[np.ndarray] = None) -> Workload:
    """Draw one workload.  ``device`` is where torch draws the tensors."""
    lens = context_lengths(cfg, seed) if lengths is None else np.asarray(lengths, np.int64)
    assert lens.shape == (cfg.batch,)
    assert (lens >= max(1, cfg.prefix_len)).all()
    nb = pool_size(cfg, lens, extra_tokens=extra_steps)
    order = free_order(nb, seed)
    hq, hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    priv = lens - cfg.prefix_len
    cu = np.zeros(cfg.batch + 1, dtype=np.int64)
    cu[1:] = np.cumsum(priv)
    q = _draw(cfg, (cfg.batch, hq, d), seed, "q", device)
    pk = _draw(cfg, (cfg.prefix_len, hkv, d), seed, "prefix_k", device)
    pv = _draw(cfg, (cfg.prefix_len, hkv, d), seed, "prefix_v", device)
    ck = _draw(cfg, (int(cu[-1]), hkv, d), seed, "k", device)
    cv = _draw(cfg, (int(cu[-1]), hkv, d), seed, "v", device)
    sk = _draw(cfg, (extra_steps, cfg.batch, hkv, d), seed, "step_k", device)
    sv = _draw(cfg, (extra_steps, cfg.batch, hkv, d), seed, "step_v", device)
    return Workload(cfg, seed, lens, nb, order, q, pk, pv, ck, cv, cu, sk, sv)


# --------------------------------------------------------------------------
# Fan-out (beam-search / parallel-sample style) workload
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class BeamConfig:
    """``groups`` prompts, each forked into ``fanout`` sequences that share it.

    Prompt lengths are uniform in [length_lo, length_hi] and usually end inside
    a block, so the first token each sharer appends copies that partly filled
    block (all but the last sharer in call order).
    """
    name: str
    groups: int
    fanout: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    length_lo: int
    length_hi: int
    pool_headroom: float = 1.25
    value_dist: str = "normal"      # N(0,1)

    @property
    def batch(self) -> int:
        return self.groups * self.fanout


BEAM_CONFIGS: Dict[str, BeamConfig] = {
    "beam": BeamConfig("beam", 64, 4, 32, 8, 128, 16, "bf16", 128, 2048),
}


@dataclasses.dataclass
class BeamWorkload:
    cfg: BeamConfig
    seed: int
    prompt_lengths: np.ndarray    # int64[groups]
    num_blocks: int
    free_order: np.ndarray        # int32[num_blocks]
    q: object                     # torch [batch, Hq, D]; sequence b belongs to group b // fanout
    prompt_k: object              # torch [sum(prompt_lengths), Hkv, D]
    prompt_v: object
    cu: np.ndarray                # int64[groups + 1] prompt offsets
    step_k: object                # torch [steps, batch, Hkv, D]
    step_v: object

    @property
    def torch_dtype(self):
        import torch
        return torch.float32 if self.cfg.dtype == "f32" else torch.bfloat16

    def seq_kv(self, b: int, steps: int):
        """(k, v) of sequence b in logical order after ``steps`` appended tokens."""
        import torch
        gi = b // self.cfg.fanout
        lo, hi = int(self.cu[gi]), int(self.cu[gi + 1])
        k = torch.cat([self.prompt_k[lo:hi], self.step_k[:steps, b]], 0)
        v = torch.cat([self.prompt_v[lo:hi], self.step_v[:steps, b]], 0)
        return k, v


def make_beam_workload(cfg: BeamConfig, seed: int = 0, device="cpu",
                       steps: int = 1) -> BeamWorkload:
    rng = _rng(seed, "lengths")
    plen = rng.integers(cfg.length_lo, cfg.length_hi + 1, size=cfg.groups, dtype=np.int64)
    p = cfg.block_size
    # prompts once, then every sequence's own blocks for its appended tokens
    # (a copied partial block plus the blocks its new tokens open)
    need = sum(_pages(int(l), p) for l in plen)
    need += sum(cfg.fanout * (_pages(int(l) + steps, p) - int(l) // p) for l in plen)
    nb = int(math.ceil(cfg.pool_headroom * need))
    order = free_order(nb, seed)
    cu = np.zeros(cfg.groups + 1, dtype=np.int64)
    cu[1:] = np.cumsum(plen)
    b = cfg.batch
    hq, hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    draw = lambda shape, stream: _draw(cfg, shape, seed, stream, device)  # noqa: E731
    return BeamWorkload(cfg, seed, plen, nb, order, draw((b, hq, d), "q"),
                        draw((int(cu[-1]), hkv, d), "k"), draw((int(cu[-1]), hkv, d), "v"), cu,
                        draw((steps, b, hkv, d), "step_k"), draw((steps, b, hkv, d), "step_v"))


# --------------------------------------------------------------------------
# Prefill (appended chunk) workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    """``batch`` sequences holding ``context`` tokens each receive ``new`` more."""
    name: str
    batch: int
    context: int
    new: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str = "bf16"
    value_dist: str = "normal"


PREFILL_CONFIGS: Dict[str, PrefillConfig] = {
    # whole prompts: 16 fresh sequences of 2048 tokens, Llama-3-8B-like heads
    "prefill": PrefillConfig("prefill", 16, 0, 2048, 32, 8, 128, 16),
    # chunked prefill: 32 sequences holding 4096 tokens append 512 more
    "prefill_chunk": PrefillConfig("prefill_chunk", 32, 4096, 512, 32, 8, 128, 16),
}


@dataclasses.dataclass
class PrefillWorkload:
    cfg: PrefillConfig
    seed: int
    num_blocks: int
    free_order: np.ndarray
    ctx_k: object      # torch [batch * context, Hkv, D], sequence-major
    ctx_v: object
    new_k: object      # torch [batch * new, Hkv, D]
    new_v: object
    q: object          # torch [batch * new, Hq, D]


def make_prefill_workload(cfg: PrefillConfig, seed: int = 0, device="cpu") -> PrefillWorkload:
    p = cfg.block_size
    nb = int(math.ceil(1.25 * cfg.batch * _pages(cfg.context + cfg.new, p)))
    hq, hkv, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    draw = lambda shape, stream: _draw(cfg, shape, seed, stream, device)  # noqa: E731
    b = cfg.batch
    return PrefillWorkload(cfg, seed, nb, free_order(nb, seed),
                           draw((b * cfg.context, hkv, d), "k"), draw((b * cfg.context, hkv, d), "v"),
                           draw((b * cfg.new, hkv, d), "new_k"), draw((b * cfg.new, hkv, d), "new_v"),
                           draw((b * cfg.new, hq, d), "q"))


@dataclasses.dataclass(frozen=True)
class AdmissionConfig:
    """A stream of requests with log-uniform prompt and output lengths.

    ``max_output`` is every request's declared output limit (what an up-front
    reservation holds room for); the drawn output length never exceeds it.
    The KV memory is ``num_blocks * block_size`` slots for both policies.
    """
    name: str
    n_requests: int
    prompt_lo: int
    prompt_hi: int
    output_lo: int
    output_hi: int
    max_output: int
    num_blocks: int
    block_size: int


ADMISSION_CONFIGS: Dict[str, AdmissionConfig] = {
    # 4096 requests, prompts and outputs log-uniform in [16, 1024], limit 2048,
    # 2^18 KV slots (16384 blocks of 16 tokens)
    "admission": AdmissionConfig("admission", 4096, 16, 1024, 16, 1024, 2048, 16384, 16),
    # a small trace the pure-Python pool model replays in seconds
    "admission_small": AdmissionConfig("admission_small", 300, 4, 200, 1, 200, 256, 512, 8),
}


def _loguniform_int(rng: np.random.Generator, lo: int, hi: int, n: int) -> np.ndarray:
    out = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi + 1), size=n))).astype(np.int64)
    return np.clip(out, lo, hi)


def make_admission_trace(cfg: AdmissionConfig, seed: int = 0):
    """(prompts, outputs, max_outputs, free_order) as int64 / int32 arrays."""
    rng = _rng(seed, "admission")
    prompts = _loguniform_int(rng, cfg.prompt_lo, cfg.prompt_hi, cfg.n_requests)
    outputs = _loguniform_int(rng, cfg.output_lo, cfg.output_hi, cfg.n_requests)
    outputs = np.minimum(outputs, cfg.max_output)
    max_outputs = np.full(cfg.n_requests, cfg.max_output, dtype=np.int64)
    return prompts, outputs, max_outputs, free_order(cfg.num_blocks, seed)
