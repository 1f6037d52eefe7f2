"""Admission of a synthetic request stream under paged blocks vs up-front reservation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
-------
* "pagedattention" topic page, paragraphs on memory waste and batching:
  reserving room for the longest possible output wastes most of the cache and
  limits how many requests run together; blocks handed out as tokens arrive
  waste at most the unfilled tail of each sequence's last block.
* "PagedAttention Internals", "Fixed-Size KV Blocks" and "Sharing And Dynamic
  Growth": a sequence takes a block only when its current one is full and
  returns its blocks when it finishes.

The pages give the capacity argument, not a scheduler.  The loop replayed here
is the plainest one that exercises it (a reading, the same one the library's
admission module states):

Each step,
  1. admit: while the first queued request fits, start it.  Paged: the free
     blocks must cover its context plus one token (context = prompt plus the
     tokens it generated before a preemption).  Reserved: the slots already
     reserved plus prompt + max_output must not exceed the capacity.
  2. generate one token for every running sequence.  Paged only: if the
     tokens that open a new block outnumber the free blocks, the most
     recently admitted running sequence is preempted (its blocks released, the
     request put back at the front of the queue), repeatedly, until they fit.
  3. every sequence that has generated its output length finishes and
     releases its memory.
Requests that could never run alone are rejected before the first step.

The paged side runs on ``PoolModel`` (this package's block pool), the
reserved side is arithmetic.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

from .pool_model import PoolModel


def _blocks(tokens: int, p: int) -> int:
    """Blocks that hold `tokens` tokens (ceiling division)."""
    return (tokens + p - 1) // p


def paged(num_blocks: int, block_size: int, prompts: Sequence[int], outputs: Sequence[int],
          free_order=None, max_steps: Optional[int] = None) -> Dict[str, object]:
    p = block_size
    pool = PoolModel(num_blocks, p, free_order)
    cap = num_blocks * p
    prompts = [int(x) for x in prompts]
    outputs = [int(x) for x in outputs]
    rejected = [i for i in range(len(prompts)) if prompts[i] + outputs[i] > cap]
    queue: List[int] = [i for i in range(len(prompts)) if i not in set(rejected)]
    generated = [0] * len(prompts)
    running: List[List[int]] = []          # [request, sequence id], admission order
    rec: Dict[str, List[int]] = {k: [] for k in
                                 ("running", "held", "live", "admitted", "finished", "preempted")}
    completed = 0
    while queue or running:
        if max_steps is not None and len(rec["running"]) >= max_steps:
            break
        admitted = 0
        while queue:
            r = queue[0]
            context = prompts[r] + generated[r]
            if len(pool.free) < _blocks(context + 1, p):
                break
            queue.pop(0)
            sid = pool.seq_create()
            pool.append_slots([sid], [context])
            running.append([r, sid])
            admitted += 1
        preempted = 0
        while True:
            opening = sum(1 for r, sid in running if pool.lengths[sid] % p == 0)
            if opening <= len(pool.free):
                break
            r, sid = running.pop()
            pool.free_seq(sid)
            queue.insert(0, r)
            preempted += 1
        if running:
            pool.append_slots([sid for _, sid in running], [1] * len(running))
        for r, _ in running:
            generated[r] += 1
        n_running = len(running)
        finished = 0
        still = []
        for r, sid in running:
            if generated[r] == outputs[r]:
                pool.free_seq(sid)
                finished += 1
            else:
                still.append([r, sid])
        running = still
        completed += finished
        st = pool.stats()
        rec["running"].append(n_running)
        rec["held"].append(st["used_blocks"] * p)
        rec["live"].append(st["live_tokens"])
        rec["admitted"].append(admitted)
        rec["finished"].append(finished)
        rec["preempted"].append(preempted)
    return {"rec": rec, "rejected": rejected, "completed": completed, "capacity_slots": cap}


def reserved(capacity_slots: int, prompts: Sequence[int], outputs: Sequence[int],
             max_outputs: Sequence[int], max_steps: Optional[int] = None) -> Dict[str, object]:
    cap = capacity_slots
    need = [int(a) + int(m) for a, m in zip(prompts, max_outputs)]
    rejected = [i for i in range(len(need)) if need[i] > cap]
    queue = [i for i in range(len(need)) if need[i] <= cap]
    generated = [0] * len(need)
    running: List[int] = []
    held = 0
    rec: Dict[str, List[int]] = {k: [] for k in
                                 ("running", "held", "live", "admitted", "finished", "preempted")}
    completed = 0
    while queue or running:
        if max_steps is not None and len(rec["running"]) >= max_steps:
            break
        admitted = 0
        while queue and held + need[queue[0]] <= cap:
            r = queue.pop(0)
            held += need[r]
            running.append(r)
            admitted += 1
        for r in running:
            generated[r] += 1
        n_running = len(running)
        finished = 0
        still = []
        for r in running:
            if generated[r] == int(outputs[r]):
                held -= need[r]
                finished += 1
            else:
                still.append(r)
        running = still
        completed += finished
        rec["running"].append(n_running)
        rec["held"].append(held)
        rec["live"].append(sum(int(prompts[r]) + generated[r] for r in running))
        rec["admitted"].append(admitted)
        rec["finished"].append(finished)
        rec["preempted"].append(0)
    return {"rec": rec, "rejected": rejected, "completed": completed, "capacity_slots": cap}
