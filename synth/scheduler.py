"""Seeded iteration-level scheduler: the continuous-batching trace that
drives one packed attention step per iteration.

Policy (from the pages; readings where they leave a choice):

* Iteration-level scheduling: after every step finished requests leave and
  waiting ones are admitted ([MLM] "连续批处理：动态调度与不规则批处理"; [YB] 11.2.2, three things per
  step; [CB] "Scheduler 的三个数据结构").
* A per-step token budget (max_num_batched_tokens): decode rows first, then
  requests still prefilling, then first-come-first-served admission of
  waiting requests, each chunked into the budget left ([YB] 11.2.5:
  the decode tokens are placed first and prefill chunks fill the rest;
  [CB] chunked prefill).
  An optional cap on running sequences (max_num_seqs) bounds concurrency.
* Paged blocks of 16 tokens from a fixed pool, allocated when a sequence
  needs a new block and all returned when it finishes ([PA] "分页设计";
  [YB] 11.2.3).
* When no block is free for a running request, recompute preemption: the
  victim's blocks go back to the pool and it returns to the head of the
  waiting queue holding prompt + generated tokens, to be prefilled again
  ([CB] "策略 B：Recompute-based"; [PA] "抢占策略").  Victim: least recently
  scheduled, ties to the most recently admitted ([CB] "Preemption 优先级":
  LRU).
* A step that finishes a request's known tokens samples one token
  ([K4I], section "与 KV cache 的关系": the step that completes a prefill
  also yields the first output token); a request is done when it
  has generated its output length (EOS at the drawn length).

A request's tokens are its prompt followed by what it generated; ``computed``
of them have K/V in the cache.  Each step processes ``q_len`` tokens starting
at ``computed``: the packed rows' cached prefix is ``computed`` and
``seq_lens = computed + q_len`` (post-append visible keys).
"""

from __future__ import annotations

import collections
import dataclasses
import math
from typing import Deque, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16


@dataclasses.dataclass
class Request:
    rid: int
    prompt_len: int
    output_len: int
    arrival_step: int = 0
    generated: int = 0
    computed: int = 0
    blocks: List[int] = dataclasses.field(default_factory=list)
    admitted_step: int = -1
    last_scheduled: int = -1
    preemptions: int = 0
    first_step: int = -1
    done_step: int = -1

    @property
    def known(self) -> int:
        return self.prompt_len + self.generated

    @property
    def decoding(self) -> bool:
        return self.known - self.computed == 1


@dataclasses.dataclass
class Step:
    index: int
    rows: List[Tuple[int, int, int]]      # (rid, cached, q_len) in packed order
    cu_seqlens_q: np.ndarray
    seq_lens: np.ndarray
    block_tables: np.ndarray
    n_decode: int
    n_prefill_rows: int
    preempted: List[int]
    finished: List[int]

    @property
    def num_rows(self) -> int:
        return int(self.cu_seqlens_q[-1])


class BlockPool:
    """Free list of physical block ids (a seeded permutation, so placement is
    random); blocks are handed out from the front and returned to the back."""

    def __init__(self, num_blocks: int, rng: Optional[np.random.Generator] = None):
        ids = np.arange(num_blocks) if rng is None else rng.permutation(num_blocks)
        self.free: Deque[int] = collections.deque(int(i) for i in ids)
        self.num_blocks = num_blocks

    def take(self, n: int) -> Optional[List[int]]:
        if n > len(self.free):
            return None
        return [self.free.popleft() for _ in range(n)]

    def give(self, blocks: Sequence[int]):
        self.free.extend(blocks)


class Scheduler:
    def __init__(self, num_blocks: int, token_budget: int, max_num_seqs: Optional[int] = None,
                 rng: Optional[np.random.Generator] = None):
        self.pool = BlockPool(num_blocks, rng)
        self.budget = token_budget
        self.max_num_seqs = max_num_seqs
        self.waiting: Deque[Request] = collections.deque()
        self.running: List[Request] = []
        self.finished: List[Request] = []
        self.step_index = 0
        self.preemptions = 0

    # ------------------------------------------------------------ helpers
    def add(self, req: Request):
        self.waiting.append(req)

    def _blocks_for(self, n_tokens: int) -> int:
        return (n_tokens + BLOCK - 1) // BLOCK

    def _grow(self, r: Request, n_tokens: int) -> bool:
        need = self._blocks_for(n_tokens) - len(r.blocks)
        if need <= 0:
            return True
        got = self.pool.take(need)
        if got is None:
            return False
        r.blocks.extend(got)
        return True

    def _preempt(self, victim: Request):
        self.pool.give(victim.blocks)
        victim.blocks = []
        victim.computed = 0
        victim.preemptions += 1
        self.preemptions += 1
        self.running = [r for r in self.running if r is not victim]
        self.waiting.appendleft(victim)

    def _victim(self, exclude) -> Optional[Request]:
        cands = [r for r in self.running if r.rid not in exclude]
        if not cands:
            return None
        return min(cands, key=lambda r: (r.last_scheduled, -r.admitted_step, -r.rid))

    # ------------------------------------------------------------ one step
    def schedule(self) -> Step:
        s = self.step_index
        rows: List[Tuple[Request, int]] = []
        taken = set()
        budget = self.budget
        preempted = []

        def place(r: Request, q_len: int) -> bool:
            """Reserve blocks for r's next q_len tokens, preempting LRU
            victims (never a request already placed in this step)."""
            while not self._grow(r, r.computed + q_len):
                v = self._victim(exclude=taken | {r.rid})
                if v is None:
                    return False
                preempted.append(v.rid)
                self._preempt(v)
            return True

        # 1. decode rows of running requests, then 2. running prefills
        for phase in ("decode", "prefill"):
            for r in list(self.running):
                if r.rid in taken or r.rid in preempted or budget <= 0:
                    continue
                if (phase == "decode") != r.decoding:
                    continue
                q_len = min(r.known - r.computed, budget)
                if not place(r, q_len):
                    # nothing left to take from: r itself waits for a later step
                    self._preempt(r)
                    preempted.append(r.rid)
                    continue
                rows.append((r, q_len))
                taken.add(r.rid)
                budget -= q_len
        # 3. FCFS admission into what is left (no preemption to admit)
        while self.waiting and budget > 0:
            if self.max_num_seqs is not None and len(self.running) >= self.max_num_seqs:
                break
            r = self.waiting[0]
            if r.rid in preempted:      # not re-admitted in the step that evicted it
                break
            q_len = min(r.known - r.computed, budget)
            if not self._grow(r, r.computed + q_len):
                break
            self.waiting.popleft()
            self.running.append(r)
            r.admitted_step = s
            if r.first_step < 0:
                r.first_step = s
            rows.append((r, q_len))
            taken.add(r.rid)
            budget -= q_len

        # packed metadata
        S = len(rows)
        cu = np.zeros(S + 1, dtype=np.int32)
        sl = np.zeros(S, dtype=np.int32)
        mb = max([self._blocks_for(r.computed + q) for r, q in rows] + [1])
        bt = np.full((S, mb), -1, dtype=np.int32)
        rec = []
        for i, (r, q) in enumerate(rows):
            cu[i + 1] = cu[i] + q
            sl[i] = r.computed + q
            nb = self._blocks_for(sl[i])
            bt[i, :nb] = r.blocks[:nb]
            rec.append((r.rid, r.computed, q))
            r.last_scheduled = s
        n_dec = sum(1 for r, q in rows if q == 1 and r.decoding)

        # the step runs; then every scheduled request advances
        finished = []
        for r, q in rows:
            r.computed += q
            if r.computed == r.known:
                r.generated += 1
                if r.generated >= r.output_len:
                    r.done_step = s
                    self.pool.give(r.blocks)
                    r.blocks = []
                    self.finished.append(r)
                    finished.append(r.rid)
        if finished:
            done = set(finished)
            self.running = [r for r in self.running if r.rid not in done]
        self.step_index += 1
        return Step(s, rec, cu, sl, bt, n_dec, int(cu[-1]) - n_dec, preempted, finished)


# ----------------------------------------------------------------------------
# the continuous-batching trace and the pages' small schedules
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class TraceConfig:
    steps: int = 200
    arrival_rate: float = 8.0      # Poisson requests per step
    prompt_min: int = 32
    prompt_max: int = 2048
    output_min: int = 10
    output_max: int = 2000
    token_budget: int = 8192
    num_blocks: int = 65536
    seed: int = 149005


def continuous_batching_trace(cfg: TraceConfig = TraceConfig()) -> Tuple[List[Step], Scheduler]:
    """200 steps of Poisson arrivals (prompt lengths uniform in [32, 2048],
    output lengths log-uniform in [10, 2000]) through the scheduler with an
    8192-token budget and a 65,536-block pool."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    sch = Scheduler(cfg.num_blocks, cfg.token_budget, rng=rng)
    steps, rid = [], 0
    for s in range(cfg.steps):
        for _ in range(int(rng.poisson(cfg.arrival_rate))):
            p = int(rng.integers(cfg.prompt_min, cfg.prompt_max, endpoint=True))
            o = int(round(math.exp(rng.uniform(math.log(cfg.output_min), math.log(cfg.output_max)))))
            sch.add(Request(rid, p, o, arrival_step=s))
            rid += 1
        steps.append(sch.schedule())
    return steps, sch


def static_batching(output_lens: Sequence[int], batch: int) -> Tuple[int, float]:
    """Steps and useful fraction of static batching: groups of ``batch`` in
    arrival order, each running until its longest member finishes ([MLM]
    "静态批处理的问题"; [YB] 11.2.1)."""
    steps = 0
    for i in range(0, len(output_lens), batch):
        steps += max(output_lens[i:i + batch])
    return steps, sum(output_lens) / (batch * steps)


def slot_schedule(output_lens: Sequence[int], slots: int) -> Tuple[int, List[int], List[int]]:
    """Continuous batching with a fixed number of slots and no token or
    memory limit: returns (steps, first step, done step) per request, steps
    numbered from 1."""
    sch = Scheduler(num_blocks=1 << 20, token_budget=1 << 30, max_num_seqs=slots)
    for i, n in enumerate(output_lens):
        sch.add(Request(i, prompt_len=1, output_len=n))
    while sch.waiting or sch.running:
        sch.schedule()
    reqs = sorted(sch.finished, key=lambda r: r.rid)
    return sch.step_index, [r.first_step + 1 for r in reqs], [r.done_step + 1 for r in reqs]
