"""Paged KV cache and paged decode attention for AMD MI355X (gfx950).

A thin binding over libpkv.so (C ABI in include/pkv.h).  Every function here
only checks and marshals arguments; all work happens in the library: the host
block pool in C++, the cache and attention kernels in HIP.  Device tensors are
torch tensors on a ROCm device (torch supplies memory and streams only).  If
libpkv.so is missing the import fails: there is no fallback path.

Names follow the pages' vocabulary: a *block pool* of fixed-size blocks, a
per-sequence *block table* from logical to physical block, *slots* inside
blocks, *fork* / copy-on-write for shared prefixes, and decode attention that
follows the table to its keys and values.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import (DEVERR_CONTEXT_LEN, DEVERR_COPY_PAIR, DEVERR_SLOT,  # noqa: F401
                   DEVERR_TABLE_ENTRY, DEVERR_WORK_OVERFLOW)

lib = _lib.load()

__all__ = ["PkvError", "BlockPool", "cache_append", "copy_blocks", "decode_workspace_bytes",
           "paged_attention_decode", "paged_attention_decode_noalloc", "decode_plan",
           "paged_attention_decode_planned", "paged_attention_prefill",
           "check_device_errors", "version", "lib", "DECODE_SCRATCH_BYTES"]


class PkvError(RuntimeError):
    """A non-zero status from libpkv.so; ``code`` is the PKV_ERR_* value."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[pkv {code}] {msg}")
        self.code = code


def _check(rc: int) -> None:
    if rc != _lib.OK:
        raise PkvError(rc, lib.pkv_last_error().decode(errors="replace"))


def version() -> str:
    return lib.pkv_version().decode()


def _i32_array(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _i64_array(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int32))


def _p64(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int64))


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return _lib.F32
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class BlockPool:
    """Host block pool (free list, refcounts, per-sequence block tables)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._h = C.c_void_p()
        order = None if free_order is None else _i32_array(free_order)
        if order is not None and order.shape != (num_blocks,):
            raise ValueError("free_order must have num_blocks entries")
        _check(lib.pkv_pool_create(num_blocks, block_size,
                                   None if order is None else _p32(order), C.byref(self._h)))
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if self._h:
            _check(lib.pkv_pool_destroy(self._h))
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def seq_create(self) -> int:
        out = C.c_int64()
        _check(lib.pkv_seq_create(self._h, C.byref(out)))
        return out.value

    def append_slots(self, seqs: Sequence[int], n_new: Sequence[int],
                     cow_cap: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Slots of the new tokens (int32, call order) and CoW pairs (int32 [n, 2])."""
        s = _i64_array(seqs)
        n = _i32_array(n_new)
        if s.shape != n.shape or s.ndim != 1:
            raise ValueError("seqs and n_new must be 1-D and of equal length")
        total = int(n.astype(np.int64).sum()) if n.size else 0
        slots = np.empty(max(total, 1), dtype=np.int32)
        cap = len(s) if cow_cap is None else int(cow_cap)
        cow = np.empty(2 * max(cap, 1), dtype=np.int32)
        ncow = C.c_int32(0)
        _check(lib.pkv_seq_append_slots(self._h, _p64(s), _p32(n), len(s), _p32(slots), total,
                                        _p32(cow), cap, C.byref(ncow)))
        return slots[:total], cow[:2 * ncow.value].reshape(-1, 2)

    def fork(self, parent: int) -> int:
        out = C.c_int64()
        _check(lib.pkv_seq_fork(self._h, int(parent), C.byref(out)))
        return out.value

    def free(self, seq: int) -> None:
        _check(lib.pkv_seq_free(self._h, int(seq)))

    def set_table(self, seq: int, phys: Sequence[int], length: int) -> None:
        p = _i32_array(phys)
        _check(lib.pkv_seq_set_table(self._h, int(seq), _p32(p), len(p), int(length)))

    def get_table(self, seq: int) -> Tuple[np.ndarray, int]:
        n = C.c_int32()
        ln = C.c_int64()
        cap = self.num_blocks
        buf = np.empty(cap, dtype=np.int32)
        _check(lib.pkv_seq_get_table(self._h, int(seq), _p32(buf), cap, C.byref(n), C.byref(ln)))
        return buf[:n.value].copy(), ln.value

    def stats(self) -> dict:
        st = _lib.Stats()
        _check(lib.pkv_pool_stats(self._h, C.byref(st)))
        return {k: getattr(st, k) for k, _ in _lib.Stats._fields_}

    def export(self) -> Tuple[np.ndarray, np.ndarray]:
        """(free list in order, refcount of every block)."""
        free = np.empty(self.num_blocks, dtype=np.int32)
        ref = np.empty(self.num_blocks, dtype=np.int32)
        nf = C.c_int32()
        _check(lib.pkv_pool_export(self._h, _p32(free), _p32(ref), C.byref(nf)))
        return free[:nf.value].copy(), ref

    def shared_prefix(self, seqs: Sequence[int]) -> Tuple[np.ndarray, int]:
        """(tokens each sequence holds in the previous one's blocks, unshared total)."""
        s = _i64_array(seqs)
        sh = np.empty(max(len(s), 1), dtype=np.int32)
        un = C.c_int64()
        _check(lib.pkv_seq_shared_prefix(self._h, _p64(s), len(s), _p32(sh), C.byref(un)))
        return sh[:len(s)].copy(), un.value

    def block_table_upload(self, seqs: Sequence[int], max_blocks: int, d_block_table,
                           d_context_lens, slot_mapping=None, d_slot_mapping=None,
                           stream=None, incremental: bool = False,
                           d_shared_prev=None) -> Tuple[int, int]:
        """Upload the padded block table and lengths; returns (max length, total tokens).

        ``incremental=True`` sends only what changed since this pool's last upload
        to the same device table (see PKV_UPLOAD_INCREMENTAL in pkv.h).
        ``d_shared_prev`` (device int32 [n_seqs], optional) receives, per
        sequence, the leading tokens it holds in the previous sequence's blocks.
        """
        import torch
        s = _i64_array(seqs)
        if d_block_table.dtype != torch.int32 or d_context_lens.dtype != torch.int32:
            raise TypeError("block table and lengths must be int32")
        if d_block_table.numel() < len(s) * max_blocks or d_context_lens.numel() < len(s):
            raise ValueError("device buffers too small")
        if d_shared_prev is not None and (d_shared_prev.dtype != torch.int32 or
                                          d_shared_prev.numel() < len(s)):
            raise ValueError("d_shared_prev must be an int32 device tensor of n_seqs entries")
        n_slots = 0
        hs = None
        if slot_mapping is not None:
            hs = _i32_array(slot_mapping)
            n_slots = len(hs)
            if d_slot_mapping is None or d_slot_mapping.numel() < n_slots or \
                    d_slot_mapping.dtype != torch.int32:
                raise ValueError("d_slot_mapping must be an int32 device tensor large enough")
        mx = C.c_int32()
        tot = C.c_int64()
        _check(lib.pkv_block_table_upload(
            self._h, _p64(s), len(s), int(max_blocks), _dev(d_block_table, "block table"),
            _dev(d_context_lens, "context lengths"),
            None if d_shared_prev is None else _dev(d_shared_prev, "shared tokens"),
            None if hs is None else _p32(hs),
            None if hs is None else _dev(d_slot_mapping, "slot mapping"), n_slots,
            C.byref(mx), C.byref(tot), _lib.UPLOAD_INCREMENTAL if incremental else 0,
            _stream_ptr(stream)))
        return mx.value, tot.value


LAYOUTS = {"head_major": _lib.LAYOUT_HEAD_MAJOR, "token_major": _lib.LAYOUT_TOKEN_MAJOR}


def _cache_shape(k_cache, v_cache, layout="head_major"):
    """(num_blocks, Hkv, block_size, D, layout code); the value cache fixes the sizes."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    if k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("k_cache and v_cache must be 4-D")
    nb, hkv, d, bs = v_cache.shape
    want = (nb, bs, hkv, d) if layout == "token_major" else (nb, hkv, bs, d)
    if tuple(k_cache.shape) != want:
        raise ValueError(f"k_cache must be {want} for layout {layout!r} "
                         "(v_cache is [num_blocks, num_kv_heads, head_dim, block_size])")
    if v_cache.dtype != k_cache.dtype:
        raise TypeError("k_cache and v_cache dtypes differ")
    return nb, hkv, bs, d, LAYOUTS[layout]


def copy_blocks(k_cache, v_cache, pairs, stream=None, layout="head_major") -> None:
    """Copy-on-write copies: pairs is host int [n, 2] of (src, dst) blocks."""
    p = _i32_array(pairs).reshape(-1)
    if p.size == 0:
        return
    nb, hkv, bs, d, _ = _cache_shape(k_cache, v_cache, layout)
    _check(lib.pkv_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _p32(p),
                               p.size // 2, nb, hkv, d, bs, _dtype_code(k_cache),
                               _stream_ptr(stream)))


def cache_append(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None,
                 layout="head_major") -> None:
    """Write k_new/v_new [n, Hkv, D] at the device int32 slots (negative = skip)."""
    import torch
    nb, hkv, bs, d, lay = _cache_shape(k_cache, v_cache, layout)
    n = k_new.shape[0]
    if tuple(k_new.shape) != (n, hkv, d) or tuple(v_new.shape) != (n, hkv, d):
        raise ValueError("k_new / v_new must be [n_tokens, num_kv_heads, head_dim]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("k_new / v_new dtype must match the cache")
    if slot_mapping.dtype != torch.int32 or slot_mapping.numel() < n:
        raise ValueError("slot_mapping must be an int32 device tensor with n entries")
    _check(lib.pkv_cache_append(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                _dev(slot_mapping, "slot_mapping"), n, nb, hkv, d, bs,
                                _dtype_code(k_cache), lay, _stream_ptr(stream)))


def decode_workspace_bytes(n_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           block_size: int, max_context_len: int, total_context_tokens: int = -1,
                           dtype=None, unshared_context_tokens: int = -1) -> int:
    import torch
    dt = _lib.BF16 if dtype in (None, torch.bfloat16) else _lib.F32
    out = C.c_size_t()
    _check(lib.pkv_decode_workspace_bytes(n_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                          max_context_len, total_context_tokens,
                                          unshared_context_tokens, dt, C.byref(out)))
    return out.value


def _decode_common(out, q, k_cache, v_cache, block_table, context_lens, shared_prev, layout):
    """Checks shared by both decode calls; returns (b, hq, hkv, d, bs, nb, layout code)."""
    import torch
    nb, hkv, bs, d, lay = _cache_shape(k_cache, v_cache, layout)
    b, hq, d2 = q.shape
    if d2 != d or tuple(out.shape) != (b, hq, d):
        raise ValueError("q / out must be [n_seqs, num_q_heads, head_dim]")
    if q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise TypeError("q / out dtype must match the cache")
    if block_table.dim() != 2 or block_table.shape[0] != b or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 [n_seqs, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or context_lens.numel() != b:
        raise ValueError("context_lens must be int32 [n_seqs]")
    if shared_prev is not None and (shared_prev.dtype != torch.int32 or shared_prev.numel() != b):
        raise ValueError("shared_prev must be int32 [n_seqs]")
    return b, hq, hkv, d, bs, nb, lay


def paged_attention_decode(out, q, k_cache, v_cache, block_table, context_lens,
                           max_context_len: int, total_context_tokens: int = -1,
                           scale: Optional[float] = None, workspace=None, stream=None,
                           layout="head_major", shared_prev=None,
                           unshared_context_tokens: int = -1):
    """Decode attention over the paged cache; writes ``out`` [B, Hq, D] and returns it.

    ``workspace`` is a uint8 device tensor of at least decode_workspace_bytes(...)
    bytes; if None one is allocated with torch (plumbing only).  ``shared_prev``
    (device int32 [B], as block_table_upload writes it) lets sequences that
    share blocks read them once per pack; the output is the same.
    ``scale`` None means 1 / sqrt(head_dim), chosen by the library.
    """
    import torch
    b, hq, hkv, d, bs, nb, lay = _decode_common(out, q, k_cache, v_cache, block_table,
                                                context_lens, shared_prev, layout)
    need = decode_workspace_bytes(b, hq, hkv, d, bs, max_context_len, total_context_tokens,
                                  q.dtype, unshared_context_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    _check(lib.pkv_paged_attention_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), _dev(context_lens, "context_lens"),
        None if shared_prev is None else _dev(shared_prev, "shared_prev"), b, hq, hkv, d, bs,
        nb, block_table.shape[1], int(max_context_len), int(total_context_tokens),
        int(unshared_context_tokens), 0.0 if scale is None else float(scale),
        _dtype_code(q), lay, _dev(workspace, "workspace"), workspace.numel(),
        _stream_ptr(stream)))
    return out


def decode_plan(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, max_blocks_per_seq: int, max_context_len: int,
                total_context_tokens: int = -1, workspace=None, dtype=None, stream=None,
                shared_prev=None, unshared_context_tokens: int = -1):
    """The plan kernel of a decode alone: writes the unit list for these sizing
    arguments and the current context lengths into ``workspace`` (required),
    for paged_attention_decode_planned calls with the same arguments."""
    import torch
    if workspace is None:
        raise ValueError("decode_plan needs the workspace the planned decode will use")
    if context_lens.dtype != torch.int32:
        raise ValueError("context_lens must be int32 [n_seqs]")
    b = context_lens.numel()
    if shared_prev is not None and (shared_prev.dtype != torch.int32 or shared_prev.numel() != b):
        raise ValueError("shared_prev must be int32 [n_seqs]")
    dt = torch.bfloat16 if dtype is None else dtype
    need = decode_workspace_bytes(b, num_q_heads, num_kv_heads, head_dim, block_size,
                                  max_context_len, total_context_tokens, dt,
                                  unshared_context_tokens)
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    code = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}.get(dt)
    if code is None:
        raise TypeError(f"unsupported dtype {dt}")
    _check(lib.pkv_decode_plan(
        _dev(context_lens, "context_lens"),
        None if shared_prev is None else _dev(shared_prev, "shared_prev"), b, int(num_q_heads),
        int(num_kv_heads), int(head_dim), int(block_size), int(max_blocks_per_seq),
        int(max_context_len), int(total_context_tokens), int(unshared_context_tokens), code,
        _dev(workspace, "workspace"), workspace.numel(), _stream_ptr(stream)))


def paged_attention_decode_planned(out, q, k_cache, v_cache, block_table, context_lens,
                                   max_context_len: int, total_context_tokens: int = -1,
                                   scale: Optional[float] = None, workspace=None, stream=None,
                                   layout="head_major", shared_prev=None,
                                   unshared_context_tokens: int = -1):
    """paged_attention_decode without its plan kernel: ``workspace`` (required)
    holds the plan decode_plan wrote for the same sizing arguments and lengths."""
    if workspace is None:
        raise ValueError("a planned decode needs the workspace decode_plan wrote")
    b, hq, hkv, d, bs, nb, lay = _decode_common(out, q, k_cache, v_cache, block_table,
                                                context_lens, shared_prev, layout)
    need = decode_workspace_bytes(b, hq, hkv, d, bs, max_context_len, total_context_tokens,
                                  q.dtype, unshared_context_tokens)
    if workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    _check(lib.pkv_paged_attention_decode_planned(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), _dev(context_lens, "context_lens"),
        None if shared_prev is None else _dev(shared_prev, "shared_prev"), b, hq, hkv, d, bs,
        nb, block_table.shape[1], int(max_context_len), int(total_context_tokens),
        int(unshared_context_tokens), 0.0 if scale is None else float(scale),
        _dtype_code(q), lay, _dev(workspace, "workspace"), workspace.numel(),
        _stream_ptr(stream)))
    return out


DECODE_SCRATCH_BYTES = _lib.DECODE_SCRATCH_BYTES


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_table, context_lens,
                                   max_context_len: int, total_context_tokens: int = -1,
                                   scale: Optional[float] = None, stream=None,
                                   layout="head_major", shared_prev=None,
                                   unshared_context_tokens: int = -1):
    """paged_attention_decode on the library's static scratch: no device allocation
    anywhere in the call.  Batches needing more than DECODE_SCRATCH_BYTES of
    workspace are refused; calls that may overlap on one device race."""
    b, hq, hkv, d, bs, nb, lay = _decode_common(out, q, k_cache, v_cache, block_table,
                                                context_lens, shared_prev, layout)
    _check(lib.pkv_paged_attention_decode_noalloc(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), _dev(context_lens, "context_lens"),
        None if shared_prev is None else _dev(shared_prev, "shared_prev"), b, hq, hkv, d, bs,
        nb, block_table.shape[1], int(max_context_len), int(total_context_tokens),
        int(unshared_context_tokens), 0.0 if scale is None else float(scale),
        _dtype_code(q), lay, _stream_ptr(stream)))
    return out


def paged_attention_prefill(out, q, k_cache, v_cache, block_table, context_lens, query_start,
                            max_query_len: int, scale: Optional[float] = None, stream=None,
                            layout="head_major"):
    """Causal attention of each sequence's newest tokens over its whole paged context.

    ``q`` / ``out`` are [total new tokens, Hq, D]; ``query_start`` is a device
    int32 [n_seqs + 1] prefix of new-token counts; the new tokens must already
    be in the cache.  Writes ``out`` and returns it.
    """
    import torch
    nb, hkv, bs, d, lay = _cache_shape(k_cache, v_cache, layout)
    nt, hq, d2 = q.shape
    if d2 != d or tuple(out.shape) != (nt, hq, d):
        raise ValueError("q / out must be [tokens, num_q_heads, head_dim]")
    if q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise TypeError("q / out dtype must match the cache")
    b = context_lens.numel()
    if block_table.dim() != 2 or block_table.shape[0] != b or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 [n_seqs, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or query_start.dtype != torch.int32 or \
            query_start.numel() != b + 1:
        raise ValueError("context_lens int32 [n_seqs], query_start int32 [n_seqs + 1]")
    _check(lib.pkv_paged_attention_prefill(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table"), _dev(context_lens, "context_lens"),
        _dev(query_start, "query_start"), b, hq, hkv, d, bs, nb, block_table.shape[1],
        int(max_query_len), 0.0 if scale is None else float(scale), _dtype_code(q), lay,
        _stream_ptr(stream)))
    return out


def check_device_errors(stream=None) -> int:
    """Synchronise and return (and clear) the device error bits; raises if any is set."""
    flags = C.c_int32(0)
    rc = lib.pkv_check_device_errors(_stream_ptr(stream), C.byref(flags))
    if rc == _lib.ERR_DEVICE:
        raise PkvError(rc, lib.pkv_last_error().decode(errors="replace") +
                       f" (flags {flags.value:#x})")
    _check(rc)
    return flags.value
