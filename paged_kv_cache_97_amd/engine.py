"""One-GPU step driver: runs the scheduler's plans through the library.

Each step (gaoleia.github.io "PagedAttention 和 Continuous Batching" §2.3-§2.6;
5688vip.com "vLLM核心机制" §3.3): the scheduler picks the rows; the engine
moves swapped blocks (pkv_swap_blocks), then either runs pkv_decode_step
(every row a single token: the new K/V are written inside the decode
attention launch) or writes the rows' new K/V into the paged pools
(pkv_write_new_tokens) and runs pkv_paged_attention_varlen.  There is no
model: every request's query, key and value rows are seeded synthetic values
that depend only on (seed, request, position) -- a gather from a
device-resident token bank -- so a token recomputed after a preemption gets
the same K/V.  The path's work runs
in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import ops
from . import workloads as W
from .scheduler import Scheduler, SchedulerConfig, StepPlan


@dataclass
class StepOutput:
    plan: StepPlan
    out: Optional[torch.Tensor]          # float32 [num_tokens, Hq, D], rows in plan order
    query_start_loc: Optional[np.ndarray]


class Engine:
    def __init__(self, config: SchedulerConfig, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 seed: int = 0, kv_cache_dtype: str = "bf16", k_scale: float = 0.0125, v_scale: float = 0.02,
                 device="cuda:0", gpu_order=None):
        if kv_cache_dtype not in ("bf16", "fp8"):
            raise ValueError("kv_cache_dtype must be 'bf16' or 'fp8'")
        self.cfg = config
        self.sched = Scheduler(config, gpu_order)
        self.Hq, self.Hkv, self.D = num_q_heads, num_kv_heads, head_dim
        self.seed = seed
        self.kv = kv_cache_dtype
        self.k_scale, self.v_scale = k_scale, v_scale
        self.scale = 1.0 / float(np.sqrt(head_dim))
        self.dev = torch.device(device)
        shape = (config.num_gpu_blocks, config.block_size, num_kv_heads, head_dim)
        pool_dtype = torch.uint8 if kv_cache_dtype == "fp8" else torch.bfloat16
        self.key_cache = torch.empty(shape, dtype=pool_dtype, device=self.dev)
        self.value_cache = torch.empty(shape, dtype=pool_dtype, device=self.dev)
        self.cpu_key = self.cpu_value = None
        if config.num_cpu_blocks > 0:
            cshape = (config.num_cpu_blocks,) + shape[1:]
            self.cpu_key = torch.empty(cshape, dtype=pool_dtype, pin_memory=True)
            self.cpu_value = torch.empty(cshape, dtype=pool_dtype, pin_memory=True)
        self.bank = W.TokenBank(seed, 8192, num_q_heads, num_kv_heads, head_dim, "bf16")
        self._bq, self._bk, self._bv = (torch.from_numpy(a).view(torch.bfloat16).to(self.dev)
                                        for a in (self.bank.q, self.bank.k, self.bank.v))
        ops.lib()                                     # fail loudly without the library

    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int) -> None:
        self.sched.add_request(req_id, prompt_len, max_new_tokens)

    def has_work(self) -> bool:
        return self.sched.has_work()

    # ------------------------------------------------------------------ one step
    def step_inputs(self, plan: StepPlan):
        """Host arrays of the plan's rows: block tables (padded with -1),
        positions, query_start_loc, seq_lens and the token-bank rows."""
        rows = plan.rows
        B = len(rows)
        width = max(1, max(len(r.block_table) for r in rows))
        bt = np.full((B, width), -1, np.int32)
        for i, r in enumerate(rows):
            bt[i, :len(r.block_table)] = r.block_table
        starts = np.fromiter((r.start for r in rows), np.int64, B)
        counts = np.fromiter((r.num_tokens for r in rows), np.int64, B)
        rids = np.fromiter((r.req_id for r in rows), np.int64, B)
        qsl = np.zeros(B + 1, np.int32)
        np.cumsum(counts, out=qsl[1:])
        sl = (starts + counts).astype(np.int32)
        T = int(qsl[-1])
        pos = (np.arange(T) + np.repeat(starts - qsl[:-1], counts)).astype(np.int32)
        idx = self.bank.index(np.repeat(rids, counts), pos)
        return bt, pos, qsl, sl, idx

    def _swap(self, pairs, to_cpu: bool) -> None:
        m = torch.tensor(pairs, dtype=torch.int64, device=self.dev)
        if to_cpu:
            ops.swap_blocks(self.key_cache, self.value_cache, self.cpu_key, self.cpu_value, m)
        else:
            ops.swap_blocks(self.cpu_key, self.cpu_value, self.key_cache, self.value_cache, m)

    def step(self) -> StepOutput:
        plan = self.sched.schedule()
        if plan.swap_out:
            self._swap(plan.swap_out, True)
        if plan.swap_in:
            self._swap(plan.swap_in, False)
        if not plan.rows:
            self.sched.complete(plan)
            return StepOutput(plan, None, None)
        bt, pos, qsl, sl, idx = self.step_inputs(plan)
        # one pinned staging buffer and one asynchronous upload per step, so
        # the host can plan the next step while this one runs
        parts = (bt.reshape(-1), pos, qsl, sl, idx.astype(np.int32))
        sizes = [a.size for a in parts]
        stage = torch.empty(sum(sizes), dtype=torch.int32, pin_memory=True)
        np.concatenate(parts, out=stage.numpy())
        flat = stage.to(self.dev, non_blocking=True)
        tbt, tpos, tqsl, tsl, tidx = torch.split(flat, sizes)
        tbt = tbt.view(bt.shape)
        tq, tk, tv = self._bq[tidx], self._bk[tidx], self._bv[tidx]
        bs = self.cfg.block_size
        max_q = int(np.diff(qsl).max())
        max_len = int(sl.max())
        if max_q == 1:
            # every row is one decode token at position seq_len - 1: one call
            # writes the new K/V and attends
            if self.kv == "fp8":
                out = ops.decode_step_fp8(tq, tk, tv, self.key_cache, self.value_cache, tbt, tsl, self.scale,
                                          max_len, self.k_scale, self.v_scale)
            else:
                out = ops.decode_step(tq, tk, tv, self.key_cache, self.value_cache, tbt, tsl, self.scale, max_len)
        elif self.kv == "fp8":
            ops.write_new_tokens_fp8(tbt, tpos, tqsl, bs, tk, tv, self.key_cache, self.value_cache, self.k_scale,
                                     self.v_scale)
            out = ops.paged_attention_varlen_fp8(tq, self.key_cache, self.value_cache, tbt, tsl, tqsl, self.scale,
                                                 max_q, max_len, self.k_scale, self.v_scale)
        else:
            ops.write_new_tokens(tbt, tpos, tqsl, bs, tk, tv, self.key_cache, self.value_cache)
            out = ops.paged_attention_varlen(tq, self.key_cache, self.value_cache, tbt, tsl, tqsl, self.scale,
                                             max_q, max_len)
        self.sched.complete(plan)
        return StepOutput(plan, out, qsl)
