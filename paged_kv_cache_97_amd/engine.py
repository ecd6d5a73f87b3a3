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
from .native_scheduler import NativeScheduler, NativeStepPlan
from .scheduler import Scheduler, SchedulerConfig, StepPlan


@dataclass
class StepOutput:
    plan: StepPlan
    # float32 [num_tokens, Hq, D], rows in plan order; a view of the engine's
    # output buffer, valid until the next step
    out: Optional[torch.Tensor]
    query_start_loc: Optional[np.ndarray]


class Engine:
    def __init__(self, config: SchedulerConfig, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 seed: int = 0, kv_cache_dtype: str = "bf16", k_scale: float = 0.0125, v_scale: float = 0.02,
                 device="cuda:0", gpu_order=None, scheduler: str = "native"):
        if kv_cache_dtype not in ("bf16", "fp8"):
            raise ValueError("kv_cache_dtype must be 'bf16' or 'fp8'")
        if scheduler not in ("native", "python"):
            raise ValueError("scheduler must be 'native' or 'python'")
        self.cfg = config
        # the native scheduler makes the same decisions as the Python one (the
        # tests compare their plans) at a fraction of the host time per step
        self.sched = (NativeScheduler if scheduler == "native" else Scheduler)(config, gpu_order)
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
        L = ops.lib()                                 # fail loudly without the library
        # Buffers that live as long as the engine, sized for the step budgets:
        # the step's query/key/value rows and output, the attention workspace
        # (the largest any step can need), and two pinned staging buffers for
        # the per-step index upload, each reused once its last copy is done.
        T = config.max_num_batched_tokens
        self._tq = torch.empty(T, num_q_heads, head_dim, dtype=torch.bfloat16, device=self.dev)
        self._tk = torch.empty(T, num_kv_heads, head_dim, dtype=torch.bfloat16, device=self.dev)
        self._tv = torch.empty_like(self._tk)
        self._out = torch.empty(T, num_q_heads, head_dim, dtype=torch.float32, device=self.dev)
        pool_kind = ops.PKV_FP8_E4M3 if kv_cache_dtype == "fp8" else ops.PKV_BF16
        B = config.max_num_seqs
        ws = max(int(L.pkv_varlen_workspace_size(B, T, num_q_heads, num_kv_heads, head_dim,
                                                 min(config.max_prefill_chunk, T), config.block_size, pool_kind)),
                 int(L.pkv_decode_workspace_size(B, num_q_heads, num_kv_heads, head_dim, config.block_size,
                                                 pool_kind)))
        if ws <= 0:
            raise ValueError("shape not supported by the library")
        self._ws = torch.zeros(ws, dtype=torch.uint8, device=self.dev)   # a new workspace starts zero-filled
        self._stage = [None, None]
        self._stage_done = [None, None]
        self._dstage = None
        self._turn = 0

    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int) -> None:
        self.sched.add_request(req_id, prompt_len, max_new_tokens)

    def has_work(self) -> bool:
        return self.sched.has_work()

    # ------------------------------------------------------------------ one step
    def step_inputs(self, plan: StepPlan):
        """Host arrays of the plan's rows: block tables (padded with -1),
        positions, query_start_loc, seq_lens and the token-bank rows."""
        if isinstance(plan, NativeStepPlan):
            idx = self.bank.index(np.repeat(plan.req_id, plan.row_tokens), plan.positions)
            return plan.block_tables, plan.positions, plan.query_start_loc, plan.seq_lens, idx
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
        m = torch.as_tensor(np.asarray(pairs, dtype=np.int64).reshape(-1, 2)).to(self.dev)
        if to_cpu:
            ops.swap_blocks(self.key_cache, self.value_cache, self.cpu_key, self.cpu_value, m)
        else:
            ops.swap_blocks(self.cpu_key, self.cpu_value, self.key_cache, self.value_cache, m)

    def step(self) -> StepOutput:
        plan = self.sched.schedule()
        native = isinstance(plan, NativeStepPlan)
        swap_out = plan.swap_out_pairs if native else plan.swap_out
        swap_in = plan.swap_in_pairs if native else plan.swap_in
        if len(swap_out):
            self._swap(swap_out, True)
        if len(swap_in):
            self._swap(swap_in, False)
        if (plan.num_rows if native else len(plan.rows)) == 0:
            self.sched.complete(plan)
            return StepOutput(plan, None, None)
        bt, pos, qsl, sl, idx = self.step_inputs(plan)
        # one asynchronous upload per step from a pinned staging buffer (two
        # alternate, each reused once its last copy has finished), so the
        # host can plan the next step while this one runs
        parts = (bt.reshape(-1), pos, qsl, sl, idx.astype(np.int32))
        sizes = [a.size for a in parts]
        n = sum(sizes)
        turn = self._turn
        self._turn ^= 1
        if self._stage_done[turn] is not None:
            self._stage_done[turn].synchronize()
        if self._stage[turn] is None or self._stage[turn].numel() < n:
            self._stage[turn] = torch.empty(2 * n, dtype=torch.int32, pin_memory=True)
        if self._dstage is None or self._dstage.numel() < n:
            self._dstage = torch.empty(2 * n, dtype=torch.int32, device=self.dev)
        stage = self._stage[turn][:n]
        np.concatenate(parts, out=stage.numpy())
        flat = self._dstage[:n]
        flat.copy_(stage, non_blocking=True)
        done = torch.cuda.Event()
        done.record()
        self._stage_done[turn] = done
        tbt, tpos, tqsl, tsl, tidx = torch.split(flat, sizes)
        tbt = tbt.view(bt.shape)
        T = int(qsl[-1])
        tq, tk, tv = self._tq[:T], self._tk[:T], self._tv[:T]
        torch.index_select(self._bq, 0, tidx, out=tq)
        torch.index_select(self._bk, 0, tidx, out=tk)
        torch.index_select(self._bv, 0, tidx, out=tv)
        out_buf = self._out[:T]
        bs = self.cfg.block_size
        max_q = int(np.diff(qsl).max())
        max_len = int(sl.max())
        if max_q == 1:
            # every row is one decode token at position seq_len - 1: one call
            # writes the new K/V and attends
            if self.kv == "fp8":
                out = ops.decode_step_fp8(tq, tk, tv, self.key_cache, self.value_cache, tbt, tsl, self.scale,
                                          max_len, self.k_scale, self.v_scale, out=out_buf, workspace=self._ws)
            else:
                out = ops.decode_step(tq, tk, tv, self.key_cache, self.value_cache, tbt, tsl, self.scale, max_len,
                                      out=out_buf, workspace=self._ws)
        elif self.kv == "fp8":
            ops.write_new_tokens_fp8(tbt, tpos, tqsl, bs, tk, tv, self.key_cache, self.value_cache, self.k_scale,
                                     self.v_scale)
            out = ops.paged_attention_varlen_fp8(tq, self.key_cache, self.value_cache, tbt, tsl, tqsl, self.scale,
                                                 max_q, max_len, self.k_scale, self.v_scale, out=out_buf,
                                                 workspace=self._ws)
        else:
            ops.write_new_tokens(tbt, tpos, tqsl, bs, tk, tv, self.key_cache, self.value_cache)
            out = ops.paged_attention_varlen(tq, self.key_cache, self.value_cache, tbt, tsl, tqsl, self.scale,
                                             max_q, max_len, out=out_buf, workspace=self._ws)
        self.sched.complete(plan)
        return StepOutput(plan, out, qsl)
