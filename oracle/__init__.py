"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow reference that the GPU library is checked
against.  It is written from the three pages on PagedAttention (the
"PagedAttention Internals" lesson, the "pagedattention" topic page and the
"inference-acceleration-pagedattention-vllm" chapter) and shares no code with
the GPU path: it imports nothing from ``paged_kv_cache_399_amd`` and nothing
from the C / HIP sources.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import it; the library itself
never calls it and has no CPU fallback.

Modules
-------
``accounting``  naive-reservation vs paged fragmentation accounting.
``pool_model``  the block pool: free list, refcounts, per-sequence block
                tables, allocate-on-fill, fork / copy-on-write, release.
``layout``      slot arithmetic and the expected contents of the K and V
                caches after tokens are written at their slots.
``admission``   a synthetic request stream replayed step by step under paged
                blocks (on ``pool_model``) and under up-front reservation.
``attention``   decode attention in float64 over each sequence's keys and
                values in logical order, a pure-Python brute force for tiny
                inputs, the partition-and-merge identity for split contexts,
                and causal attention of a chunk of appended tokens (prefill).

Every function is pinned by ``tests/test_oracle_*.py`` to something other than
itself: the numbers the pages print, closed forms, brute force and library
routines.  Pins per function:

* accounting.*            printed worked examples (5 of 12 wasted, 0.417;
                          1 slot wasted under pages of 2), brute-force bounds.
* pool_model.PoolModel    printed block-table example (0,1,2 -> 8,3,11),
                          lazy allocation reproducing the 8-slot example,
                          invariants under random operation sequences.
* layout.*                round trip through the printed block table,
                          disjointness brute force.
* layout.copy_block       the copy-on-write contract on the pool model's
                          pairs (prefix of 3 in pages of 2, three sharers:
                          every sharer reads back its own tokens, blocks
                          nobody holds keep their fill), which planted
                          mistakes (swapped source and destination, keys or
                          values only, one head only) break; element-wise
                          brute force over a whole cache.
* attention.decode        brute force, torch scaled_dot_product_attention in
                          float64, closed-form two-token case, L=1 and
                          equal-key special cases, GQA == repeated MHA.
* attention.partitioned   equality with the unsplit definition.
* attention.prefill       brute force, torch scaled_dot_product_attention with an
                          explicit causal mask in float64, each row equal to
                          decode over the keys it sees, single-key rows.
* admission.*             whole-batch closed forms for identical requests
                          (reserved: cap // (prompt + limit) per wave; paged:
                          requests of whole blocks), two traces worked by hand
                          (one with preemptions), every output token generated
                          once, waste under one block per resident sequence.
"""
from . import accounting, admission, attention, layout, pool_model  # noqa: F401
from .pool_model import (PoolModel, PoolError, NoBlocks, BadSeq,  # noqa: F401
                         InvalidArg)
