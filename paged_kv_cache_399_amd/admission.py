"""Synthetic admission loop (continuous-batching style) over the block pool.

The pages' capacity argument ("pagedattention" topic page, paragraphs on
memory waste and batching; "PagedAttention Internals", "Fixed-Size KV
Blocks"): when a sequence's cache is kept in fixed-size blocks handed out as
tokens arrive, only the last block of each sequence holds unused slots, so
more sequences stay resident than when every request reserves room for its
longest possible output up front.  This module replays a synthetic request
trace step by step under both policies on the same number of KV slots:

* paged: the library's block pool (allocate on fill, free on finish);
* reserved: each admitted request holds prompt + max_output slots until it
  finishes (the up-front reservation, counted with no external
  fragmentation, which favours it).

One step of either policy:
  1. admit requests from the head of the FCFS queue while the head fits
     (paged: free blocks >= blocks for its context + 1 token; reserved:
     reserved + prompt + max_output <= capacity) — the context of a request
     preempted earlier includes the tokens it had generated;
  2. every running sequence generates one token; the paged policy first
     preempts running sequences, most recently admitted first, until the
     blocks the step needs are free (a preempted request returns to the
     queue head and is recomputed from its context when readmitted);
  3. sequences that reached their output length finish and release memory.
Requests that could not run even alone (prompt + output beyond the pool, or
prompt + max_output beyond the reservation capacity) are rejected up front.

Every step records the running count, the blocks / slots held, the live
tokens and the admissions, finishes and preemptions.  No model runs: the
generated tokens are only counted.
"""
from __future__ import annotations

import dataclasses
from collections import deque
from typing import List, Optional, Sequence

import numpy as np

from . import BlockPool


@dataclasses.dataclass
class AdmissionResult:
    running: np.ndarray        # [steps] sequences that generated a token in the step
    held: np.ndarray           # [steps] KV slots held after the step (blocks * P, or reservations)
    live: np.ndarray           # [steps] tokens stored after the step
    admitted: np.ndarray       # [steps]
    finished: np.ndarray       # [steps]
    preempted: np.ndarray      # [steps]
    rejected: List[int]        # request ids never admitted
    completed: int
    capacity_slots: int

    @property
    def steps(self) -> int:
        return int(self.running.size)

    def summary(self) -> dict:
        n = max(self.steps, 1)
        return {"steps": self.steps, "completed": self.completed, "rejected": len(self.rejected),
                "mean_running": float(self.running.sum()) / n,
                "peak_running": int(self.running.max()) if self.steps else 0,
                "generated_tokens": int(self.running.sum()),
                "preemptions": int(self.preempted.sum()),
                "mean_held_frac": float(self.held.sum()) / n / self.capacity_slots,
                "mean_live_frac": float(self.live.sum()) / n / self.capacity_slots}


def _trace(prompts, outputs, max_outputs=None):
    prompts = np.asarray(prompts, dtype=np.int64)
    outputs = np.asarray(outputs, dtype=np.int64)
    if prompts.shape != outputs.shape or prompts.ndim != 1:
        raise ValueError("prompts and outputs must be 1-D and of equal length")
    if np.any(prompts < 1) or np.any(outputs < 1):
        raise ValueError("prompt and output lengths must be >= 1")
    if max_outputs is None:
        return prompts, outputs, None
    max_outputs = np.asarray(max_outputs, dtype=np.int64)
    if max_outputs.shape != prompts.shape or np.any(max_outputs < outputs):
        raise ValueError("max_outputs must cover every output length")
    return prompts, outputs, max_outputs


def run_paged(num_blocks: int, block_size: int, prompts: Sequence[int], outputs: Sequence[int],
              free_order=None, max_steps: Optional[int] = None) -> AdmissionResult:
    """Replay the trace on a fresh library block pool."""
    prompts, outputs, _ = _trace(prompts, outputs)
    p = int(block_size)
    pool = BlockPool(num_blocks, p, free_order)
    cap = int(num_blocks) * p
    rejected = [i for i in range(prompts.size) if prompts[i] + outputs[i] > cap]
    queue = deque(i for i in range(prompts.size) if prompts[i] + outputs[i] <= cap)
    gen = np.zeros(prompts.size, dtype=np.int64)        # tokens generated so far
    run_req: List[int] = []                             # admission order
    run_seq: List[int] = []
    rec = {k: [] for k in ("running", "held", "live", "admitted", "finished", "preempted")}
    completed = 0
    free = int(num_blocks)
    try:
        while (queue or run_req) and (max_steps is None or len(rec["running"]) < max_steps):
            # 1. admission
            adm = 0
            while queue:
                r = queue[0]
                ctx = int(prompts[r] + gen[r])
                if free < -(-(ctx + 1) // p):
                    break
                queue.popleft()
                s = pool.seq_create()
                pool.append_slots([s], [ctx])
                free -= -(-ctx // p)
                run_req.append(r)
                run_seq.append(s)
                adm += 1
            # 2. generation: a token needs a new block when its context fills whole blocks
            ctxs = prompts[run_req] + gen[run_req] if run_req else np.zeros(0, np.int64)
            need = int(np.count_nonzero(ctxs % p == 0))
            pre = 0
            while need > free:
                r, s = run_req.pop(), run_seq.pop()
                c = int(prompts[r] + gen[r])
                need -= int(c % p == 0)
                free += -(-c // p)
                pool.free(s)
                queue.appendleft(r)
                pre += 1
            if run_seq:
                pool.append_slots(run_seq, np.ones(len(run_seq), np.int32))
                free -= need
                gen[run_req] += 1
            n_run = len(run_seq)
            # 3. finish
            fin = 0
            keep_r, keep_s = [], []
            for r, s in zip(run_req, run_seq):
                if gen[r] >= outputs[r]:
                    c = int(prompts[r] + gen[r])
                    free += -(-c // p)
                    pool.free(s)
                    fin += 1
                else:
                    keep_r.append(r)
                    keep_s.append(s)
            run_req, run_seq = keep_r, keep_s
            completed += fin
            st = pool.stats()
            assert st["free_blocks"] == free, "pool free count disagrees with the loop's count"
            rec["running"].append(n_run)
            rec["held"].append(int(st["used_blocks"]) * p)
            rec["live"].append(int(st["live_tokens"]))
            rec["admitted"].append(adm)
            rec["finished"].append(fin)
            rec["preempted"].append(pre)
    finally:
        pool.close()
    return AdmissionResult(**{k: np.asarray(v, dtype=np.int64) for k, v in rec.items()},
                           rejected=rejected, completed=completed, capacity_slots=cap)


def run_reserved(capacity_slots: int, prompts: Sequence[int], outputs: Sequence[int],
                 max_outputs: Sequence[int], max_steps: Optional[int] = None) -> AdmissionResult:
    """Replay the trace with prompt + max_output slots reserved per admitted request."""
    prompts, outputs, max_outputs = _trace(prompts, outputs, max_outputs)
    cap = int(capacity_slots)
    resv = prompts + max_outputs
    rejected = [i for i in range(prompts.size) if resv[i] > cap]
    queue = deque(i for i in range(prompts.size) if resv[i] <= cap)
    gen = np.zeros(prompts.size, dtype=np.int64)
    running: List[int] = []
    held = 0
    rec = {k: [] for k in ("running", "held", "live", "admitted", "finished", "preempted")}
    completed = 0
    while (queue or running) and (max_steps is None or len(rec["running"]) < max_steps):
        adm = 0
        while queue and held + resv[queue[0]] <= cap:
            r = queue.popleft()
            held += int(resv[r])
            running.append(r)
            adm += 1
        if running:
            gen[running] += 1
        n_run = len(running)
        done = [r for r in running if gen[r] >= outputs[r]]
        running = [r for r in running if gen[r] < outputs[r]]
        held -= int(resv[done].sum()) if done else 0
        completed += len(done)
        rec["running"].append(n_run)
        rec["held"].append(held)
        rec["live"].append(int((prompts[running] + gen[running]).sum()) if running else 0)
        rec["admitted"].append(adm)
        rec["finished"].append(len(done))
        rec["preempted"].append(0)
    return AdmissionResult(**{k: np.asarray(v, dtype=np.int64) for k, v in rec.items()},
                           rejected=rejected, completed=completed, capacity_slots=cap)
