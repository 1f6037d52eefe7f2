"""PagedKVCache: one layer's paged K/V cache on one device, driven step by step.

It owns a host block pool, the two device caches and the device-side metadata
(block table, context lengths, slot mapping, decode workspace), and strings the
library calls together in the order a decode step needs them:

    append_slots (host) -> copy_blocks (copy-on-write) -> block_table_upload
    (a full upload into a new table, then incremental patches of the new
    entries, lengths and slot mapping; also how many leading tokens each
    sequence holds in the previous one's blocks) -> cache_append ->
    paged_attention_decode (sequences that share blocks read them once per pack)

Everything that computes runs in libpkv.so; this class only keeps buffers and
calls the binding.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import (BlockPool, cache_append, copy_blocks, decode_plan, decode_workspace_bytes,
               paged_attention_decode, paged_attention_decode_planned, paged_attention_prefill)


def _poison_value(dtype):
    import torch
    return float("nan") if dtype in (torch.float32, torch.bfloat16) else 0


class PagedKVCache:
    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 dtype, device="cuda", free_order=None, fill: Optional[float] = None,
                 layout: str = "head_major", share_blocks: bool = True):
        import torch
        self.pool = BlockPool(num_blocks, block_size, free_order)
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.dtype, self.device = dtype, torch.device(device)
        self.layout = layout
        self.share_blocks = share_blocks
        if layout == "token_major":
            shape_k = (num_blocks, block_size, num_kv_heads, head_dim)
        elif layout == "head_major":
            shape_k = (num_blocks, num_kv_heads, block_size, head_dim)
        else:
            raise ValueError("layout must be 'head_major' or 'token_major'")
        shape_v = (num_blocks, num_kv_heads, head_dim, block_size)
        self.k_cache = torch.empty(shape_k, dtype=dtype, device=self.device)
        self.v_cache = torch.empty(shape_v, dtype=dtype, device=self.device)
        v = _poison_value(dtype) if fill is None else fill
        self.k_cache.fill_(v)
        self.v_cache.fill_(v)
        self._slots_dev = None
        self._meta = None
        self._ws = None

    # -- sequences -----------------------------------------------------------
    def new_sequences(self, n: int):
        return [self.pool.seq_create() for _ in range(n)]

    def fork(self, parent: int) -> int:
        return self.pool.fork(parent)

    def free(self, seq: int) -> None:
        self.pool.free(seq)

    def _slot_buffer(self, n: int):
        import torch
        if self._slots_dev is None or self._slots_dev.numel() < n:
            self._slots_dev = torch.empty(max(n, 1), dtype=torch.int32, device=self.device)
        return self._slots_dev

    def write(self, seqs: Sequence[int], n_new: Sequence[int], k, v, stream=None) -> np.ndarray:
        """Append tokens to sequences and store their K/V (rows in call order).

        Returns the host slot mapping.  Copy-on-write copies are enqueued
        before the write.  Uses a one-off upload of the slot mapping.
        """
        import torch
        slots, cow = self.pool.append_slots(seqs, n_new)
        if len(cow):
            copy_blocks(self.k_cache, self.v_cache, cow, stream, self.layout)
        if len(slots):
            d = torch.from_numpy(slots).to(self.device, non_blocking=False)
            cache_append(self.k_cache, self.v_cache, k, v, d, stream, self.layout)
        return slots

    def write_slots(self, slots_dev, k, v, stream=None) -> None:
        """Store rows of k/v at device slots (negative slots skip their row)."""
        cache_append(self.k_cache, self.v_cache, k, v, slots_dev, stream, self.layout)

    # -- decode step ---------------------------------------------------------
    class Meta:
        pass

    def prepare(self, seqs: Sequence[int], max_blocks: int, num_q_heads: int,
                max_context_len: int, total_tokens: int):
        """Allocate per-batch device metadata and the decode workspace once."""
        import torch
        m = self.Meta()
        m.seqs = np.asarray(seqs, dtype=np.int64)
        m.max_blocks = int(max_blocks)
        b = len(seqs)
        m.table = torch.empty((b, m.max_blocks), dtype=torch.int32, device=self.device)
        m.lens = torch.empty(b, dtype=torch.int32, device=self.device)
        m.slots = torch.empty(max(b, 1), dtype=torch.int32, device=self.device)
        m.shared = (torch.zeros(b, dtype=torch.int32, device=self.device)
                    if self.share_blocks else None)
        m.num_q_heads = num_q_heads
        m.ws_max_len = int(max_context_len)
        m.ws_total = int(total_tokens)
        # with sharing, the partition length follows the tokens left once the
        # blocks shared now are read once per pack (fixed for the batch's life)
        m.ws_unshared = -1
        if self.share_blocks and b:
            sh, _ = self.pool.shared_prefix(m.seqs)
            m.ws_unshared = max(m.ws_total - int(sh.sum()), 0)
        need = decode_workspace_bytes(b, num_q_heads, self.num_kv_heads, self.head_dim,
                                      self.block_size, m.ws_max_len, m.ws_total, self.dtype,
                                      m.ws_unshared)
        m.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=self.device)
        m.max_len = 0
        m.total = 0
        m.uploaded = False   # the first upload into this new table is a full one
        self._meta = m
        return m

    def append_decode_tokens(self, m, k_new, v_new, stream=None):
        """One decode token per sequence: host slots, CoW, upload, cache_append."""
        ones = np.ones(len(m.seqs), dtype=np.int32)
        slots, cow = self.pool.append_slots(m.seqs, ones)
        if len(cow):
            copy_blocks(self.k_cache, self.v_cache, cow, stream, self.layout)
        m.max_len, m.total = self.pool.block_table_upload(m.seqs, m.max_blocks, m.table, m.lens,
                                                          slots, m.slots, stream,
                                                          incremental=m.uploaded,
                                                          d_shared_prev=m.shared)
        m.uploaded = True
        cache_append(self.k_cache, self.v_cache, k_new, v_new, m.slots, stream, self.layout)
        return slots

    def upload(self, m, stream=None):
        """Upload table and lengths without appending (e.g. after a prefill)."""
        m.max_len, m.total = self.pool.block_table_upload(m.seqs, m.max_blocks, m.table, m.lens,
                                                          stream=stream, incremental=m.uploaded,
                                                          d_shared_prev=m.shared)
        m.uploaded = True

    def attend(self, m, q, out, scale=None, stream=None, planned=False):
        """Decode attention for the batch; planned=True reuses the plan that
        plan(m) made for the current lengths (e.g. every layer of one step)."""
        if m.max_len > m.ws_max_len or m.total > m.ws_total:
            raise ValueError("batch outgrew the workspace sized in prepare()")
        # the sizing hints stay the prepared ones, so the partition size (and
        # with it the summation order) is fixed for the life of the batch
        fn = paged_attention_decode_planned if planned else paged_attention_decode
        return fn(out, q, self.k_cache, self.v_cache, m.table, m.lens, m.ws_max_len, m.ws_total,
                  scale, m.workspace, stream, self.layout, shared_prev=m.shared,
                  unshared_context_tokens=m.ws_unshared)

    def plan(self, m, stream=None):
        """Plan the decode of the batch's current lengths once (decode_plan);
        attend(..., planned=True) then skips the plan kernel."""
        if m.max_len > m.ws_max_len or m.total > m.ws_total:
            raise ValueError("batch outgrew the workspace sized in prepare()")
        decode_plan(m.lens, m.num_q_heads, self.num_kv_heads, self.head_dim, self.block_size,
                    m.max_blocks, m.ws_max_len, m.ws_total, m.workspace, self.dtype, stream,
                    shared_prev=m.shared, unshared_context_tokens=m.ws_unshared)

    def capture_attend(self, m, q, out, scale=None):
        """Record one decode call (plan, partition, merge kernels) into a HIP graph.

        Returns a torch CUDAGraph whose replay() reruns the decode on the same
        buffers: q, out and m's table, lengths and workspace, read as they are
        at replay time (the decode allocates nothing and issues no memset or
        copy, so every replay is a pure kernel sequence).  Call attend() once
        before capturing (one-time host set-up).  The batch must stay within
        the sizing given to prepare(); replay() does not check it, call
        check_graph_sizing(m) when lengths grow.
        """
        import torch
        self.check_graph_sizing(m)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.attend(m, q, out, scale, stream=torch.cuda.current_stream())
        return g

    def check_graph_sizing(self, m):
        if m.max_len > m.ws_max_len or m.total > m.ws_total:
            raise ValueError("batch outgrew the workspace sized in prepare()")

    def extend(self, m, n_new, k_new, v_new, q, out, scale=None, stream=None):
        """Append n_new[i] tokens to m.seqs[i] and attend causally from each of them.

        Rows of k_new / v_new / q / out are the new tokens, sequence by
        sequence in m.seqs order.  Slots on the host, copy-on-write copies,
        table / length / slot upload, cache_append, then prefill attention.
        """
        import torch
        n_new = np.asarray(n_new, dtype=np.int32)
        slots, cow = self.pool.append_slots(m.seqs, n_new)
        if len(cow):
            copy_blocks(self.k_cache, self.v_cache, cow, stream, self.layout)
        if m.slots.numel() < max(len(slots), 1):
            m.slots = torch.empty(len(slots), dtype=torch.int32, device=self.device)
        m.max_len, m.total = self.pool.block_table_upload(m.seqs, m.max_blocks, m.table, m.lens,
                                                          slots, m.slots, stream,
                                                          incremental=m.uploaded,
                                                          d_shared_prev=m.shared)
        m.uploaded = True
        if len(slots):
            cache_append(self.k_cache, self.v_cache, k_new, v_new, m.slots, stream, self.layout)
        qs = np.zeros(len(n_new) + 1, dtype=np.int32)
        qs[1:] = np.cumsum(n_new)
        m.query_start = torch.from_numpy(qs).to(self.device)
        return paged_attention_prefill(out, q, self.k_cache, self.v_cache, m.table, m.lens,
                                       m.query_start, int(n_new.max()) if len(n_new) else 0,
                                       scale, stream, self.layout)

    def close(self):
        self.pool.close()
