"""Host-side continuous-batching scheduler: the step either side of the paged
attention path.  It decides, once per iteration, which requests run and how
many of their tokens, and it owns the block tables the kernels read.  Pure
Python: it never touches the device (the engine turns its plan into launches).

What it follows (the pages describe the policy, they ship no scheduler):
  * gaoleia.github.io "PagedAttention 和 Continuous Batching" §2.3 (every
    iteration: drop finished requests and free their KV, admit waiting
    requests while memory allows, then schedule prefill rows and one-token
    decode rows), §2.5 (long prompts are cut into 512-token chunks that
    interleave with decodes; max_num_batched_tokens, max_num_seqs) and §2.6
    (the step's output: scheduled requests with token counts, prefill flag
    and block table, finished and preempted ids, totals).
  * 5688vip.com "vLLM核心机制" §3.3: first come first served with a memory
    watermark (stop admitting while less than ~10 % of the blocks would stay
    free); under memory pressure a request is preempted, either swapped out
    to CPU memory or releasing its blocks to be recomputed later.
  * lakecityint.com/news/209622 §1-§2: waiting, running and swapped queues;
    FCFS admission and last-in-first-out preemption (the most recently
    admitted request is preempted first); swapped requests are resumed before
    new ones are admitted; a budget of sequences and tokens per step.
  * The fourth page's scheduler loop (remove finished, admit while free
    blocks exist for the head of WAITING, then one prefill chunk or one
    decode token per running sequence in one fused call).

Readings taken where the pages are silent: a request is scheduled as a whole
(no beam groups), so preemption by recompute is the default and swapping is a
configuration choice; running requests are served before swapped ones, and
swapped ones before waiting ones; a step that had to preempt admits nothing
new; decode rows are taken before prefill chunks inside the running list
(both in admission order); a preempted-by-recompute
request goes back to the head of the waiting queue with everything it had
computed (prompt and generated tokens) to recompute as prompt.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Deque, Dict, List, Optional, Tuple

from .blocks import BlockPool, SeqBlocks, swap_in, swap_out


@dataclass
class SchedulerConfig:
    block_size: int = 16
    num_gpu_blocks: int = 1024
    num_cpu_blocks: int = 0               # swap space (blocks); 0 disables swapping
    max_num_seqs: int = 256
    max_num_batched_tokens: int = 2048
    max_prefill_chunk: int = 512
    watermark: float = 0.1                # fraction of GPU blocks admission keeps free
    preemption: str = "recompute"         # or "swap"

    def __post_init__(self):
        if self.preemption not in ("recompute", "swap"):
            raise ValueError("preemption must be 'recompute' or 'swap'")
        if self.preemption == "swap" and self.num_cpu_blocks <= 0:
            raise ValueError("swap preemption needs num_cpu_blocks > 0")
        if min(self.block_size, self.num_gpu_blocks, self.max_num_seqs, self.max_num_batched_tokens,
               self.max_prefill_chunk) <= 0:
            raise ValueError("sizes must be positive")


@dataclass(eq=False)                      # requests compare by identity
class Request:
    """A request of prompt_len prompt tokens that generates max_new_tokens.
    Token positions 0 .. prompt_len + max_new_tokens - 1 are processed in
    order; num_computed of them have K/V in the cache."""
    req_id: int
    prompt_len: int
    max_new_tokens: int
    arrival: int = 0
    num_computed: int = 0
    table: Optional[SeqBlocks] = None
    status: str = "waiting"               # waiting | running | swapped | finished
    num_preemptions: int = 0
    recompute_to: int = 0                 # tokens computed before a recompute preemption

    @property
    def total_len(self) -> int:
        return self.prompt_len + self.max_new_tokens

    @property
    def in_prefill(self) -> bool:
        """Still feeding known tokens (the prompt, or everything computed
        before a recompute preemption)."""
        return self.num_computed < self.prefill_target

    @property
    def prefill_target(self) -> int:
        return max(self.prompt_len, self.recompute_to)

    @property
    def finished(self) -> bool:
        return self.num_computed >= self.total_len


@dataclass
class ScheduledRow:
    req_id: int
    start: int                 # first position processed this step
    num_tokens: int
    is_prefill: bool
    block_table: List[int]


@dataclass
class StepPlan:
    """One iteration: what the device must do, in order -- swap-outs, swap-ins,
    then the cache write and attention of `rows` (query_start_loc follows the
    row order)."""
    rows: List[ScheduledRow] = field(default_factory=list)
    swap_out: List[Tuple[int, int]] = field(default_factory=list)   # (gpu block, cpu block)
    swap_in: List[Tuple[int, int]] = field(default_factory=list)    # (cpu block, gpu block)
    finished_ids: List[int] = field(default_factory=list)
    preempted_ids: List[int] = field(default_factory=list)

    @property
    def num_tokens(self) -> int:
        return sum(r.num_tokens for r in self.rows)

    @property
    def num_prefill(self) -> int:
        return sum(1 for r in self.rows if r.is_prefill)

    @property
    def num_decode(self) -> int:
        return sum(1 for r in self.rows if not r.is_prefill)


class Scheduler:
    def __init__(self, config: SchedulerConfig, gpu_order=None):
        self.cfg = config
        self.gpu = BlockPool(config.num_gpu_blocks, gpu_order)
        self.cpu = BlockPool(config.num_cpu_blocks) if config.num_cpu_blocks > 0 else None
        self.waiting: Deque[Request] = deque()
        self.running: List[Request] = []
        self.swapped: Deque[Request] = deque()
        self.requests: Dict[int, Request] = {}
        self._arrivals = 0

    # ---------------------------------------------------------------- queue
    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int) -> Request:
        if req_id in self.requests:
            raise ValueError("duplicate request id %d" % req_id)
        if prompt_len <= 0 or max_new_tokens <= 0:
            raise ValueError("prompt_len and max_new_tokens must be positive")
        need = -(-(prompt_len + max_new_tokens) // self.cfg.block_size)
        if need > self.cfg.num_gpu_blocks:
            raise ValueError("request %d needs %d blocks, the pool has %d" % (req_id, need, self.cfg.num_gpu_blocks))
        r = Request(req_id, prompt_len, max_new_tokens, arrival=self._arrivals)
        self._arrivals += 1
        self.requests[req_id] = r
        self.waiting.append(r)
        return r

    def has_work(self) -> bool:
        return bool(self.waiting or self.running or self.swapped)

    # ---------------------------------------------------------------- helpers
    def _blocks_needed(self, r: Request, n: int) -> int:
        have = len(r.table.mapping) if r.table else 0
        return max(0, -(-(r.num_computed + n) // self.cfg.block_size) - have)

    def _watermark_blocks(self) -> int:
        return int(self.cfg.watermark * self.cfg.num_gpu_blocks)

    def _preempt(self, victim: Request, plan: StepPlan) -> None:
        """Last-in-first-out preemption of a running request."""
        self.running.remove(victim)
        victim.num_preemptions += 1
        plan.preempted_ids.append(victim.req_id)
        if self.cfg.preemption == "swap" and self.cpu.num_free() >= len(victim.table.mapping):
            plan.swap_out += swap_out(victim.table, self.gpu, self.cpu)
            victim.status = "swapped"
            self.swapped.append(victim)
            return
        # recompute: drop the KV, keep the token count to recompute as prompt
        victim.recompute_to = max(victim.recompute_to, victim.num_computed)
        victim.table.release(self.gpu)
        victim.table = None
        victim.num_computed = 0
        victim.status = "waiting"
        self.waiting.appendleft(victim)

    def _tokens_for(self, r: Request, budget_tokens: int) -> int:
        if r.in_prefill:
            return min(self.cfg.max_prefill_chunk, r.prefill_target - r.num_computed, budget_tokens)
        return min(1, budget_tokens)

    # ---------------------------------------------------------------- step
    def schedule(self) -> StepPlan:
        cfg = self.cfg
        plan = StepPlan()
        # 1. finished requests leave and free their blocks
        for r in [r for r in self.running if r.finished]:
            self.running.remove(r)
            r.table.release(self.gpu)
            r.table = None
            r.status = "finished"
            plan.finished_ids.append(r.req_id)

        budget_tokens = cfg.max_num_batched_tokens
        budget_seqs = cfg.max_num_seqs
        grants: List[Tuple[Request, int]] = []

        # 2. running requests: decodes first, then prefill chunks, each in
        #    admission order; make room by preempting the newest running ones
        order = sorted(self.running, key=lambda r: (r.in_prefill, r.arrival))
        running = set(map(id, self.running))
        granted = set()
        for r in order:
            if id(r) not in running:
                continue                                   # preempted while making room
            if budget_seqs == 0 or budget_tokens == 0:
                break
            n = self._tokens_for(r, budget_tokens)
            need = self._blocks_needed(r, n)
            while self.gpu.num_free() < need:
                victims = [v for v in self.running if v is not r and id(v) not in granted]
                victim = max(victims, key=lambda v: v.arrival) if victims else None
                if victim is None or victim.arrival < r.arrival:
                    victim = r                              # r itself is the newest: it yields
                self._preempt(victim, plan)
                running.discard(id(victim))
                if victim is r:
                    break
            if id(r) not in running:
                continue
            r.table.append_tokens(n, self.gpu)
            grants.append((r, n))
            granted.add(id(r))
            budget_tokens -= n
            budget_seqs -= 1

        # 3. swapped requests come back (FIFO) while memory and budget allow
        while self.swapped and budget_seqs > 0 and budget_tokens > 0:
            r = self.swapped[0]
            n = self._tokens_for(r, budget_tokens)
            blocks = len(r.table.mapping) + self._blocks_needed(r, n)
            if self.gpu.num_free() - blocks < self._watermark_blocks():
                break
            self.swapped.popleft()
            plan.swap_in += swap_in(r.table, self.cpu, self.gpu)
            r.status = "running"
            self.running.append(r)
            r.table.append_tokens(n, self.gpu)
            grants.append((r, n))
            budget_tokens -= n
            budget_seqs -= 1

        # 4. waiting requests are admitted (FCFS) above the watermark (an idle
        #    engine admits its first request whatever the watermark says)
        while (self.waiting and not self.swapped and not plan.preempted_ids and budget_seqs > 0
               and budget_tokens > 0):
            r = self.waiting[0]
            n = self._tokens_for(r, budget_tokens)
            blocks = -(-n // cfg.block_size)
            floor = self._watermark_blocks() if self.running else 0
            if self.gpu.num_free() - blocks < floor:
                break
            self.waiting.popleft()
            r.table = SeqBlocks(cfg.block_size)
            r.table.append_tokens(n, self.gpu)
            r.status = "running"
            self.running.append(r)
            grants.append((r, n))
            budget_tokens -= n
            budget_seqs -= 1

        # rows in a fixed order: decode rows first, then prefill chunks
        for r, n in sorted(grants, key=lambda g: (g[0].in_prefill or g[1] > 1, g[0].arrival)):
            plan.rows.append(ScheduledRow(r.req_id, r.num_computed, n, r.in_prefill or n > 1,
                                          list(r.table.mapping)))
        return plan

    def complete(self, plan: StepPlan) -> None:
        """The device has processed `plan`: advance every scheduled request."""
        for row in plan.rows:
            r = self.requests[row.req_id]
            assert r.num_computed == row.start
            r.num_computed += row.num_tokens
            # the table now covers exactly the computed tokens
            assert r.table.num_tokens == r.num_computed
