"""Binding of the native scheduler in libpagedkv.so (include/pkv_sched.h).

Same interface and the same decisions as scheduler.Scheduler (the native code
follows that policy step for step; tests compare their plans), but planning a
step costs microseconds instead of a Python loop over requests.  A plan comes
back as NumPy arrays that the engine uploads directly: block tables padded
with -1, per-token positions, query_start_loc and seq_lens.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Tuple

import numpy as np

from . import ops
from .scheduler import ScheduledRow, SchedulerConfig

_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)
_U8P = ctypes.POINTER(ctypes.c_uint8)


class _Config(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("num_gpu_blocks", ctypes.c_int32),
                ("num_cpu_blocks", ctypes.c_int32), ("max_num_seqs", ctypes.c_int32),
                ("max_num_batched_tokens", ctypes.c_int32), ("max_prefill_chunk", ctypes.c_int32),
                ("watermark", ctypes.c_double), ("preemption_swap", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32), ("num_tokens", ctypes.c_int32), ("req_id", _I64P),
                ("start", _I32P), ("row_tokens", _I32P), ("is_prefill", _U8P), ("table_width", ctypes.c_int32),
                ("block_tables", _I32P), ("positions", _I32P), ("query_start_loc", _I32P), ("seq_lens", _I32P),
                ("num_swap_out", ctypes.c_int32), ("swap_out", _I32P), ("num_swap_in", ctypes.c_int32),
                ("swap_in", _I32P), ("num_finished", ctypes.c_int32), ("finished_ids", _I64P),
                ("num_preempted", ctypes.c_int32), ("preempted_ids", _I64P)]


def _arr(ptr, n: int, dtype) -> np.ndarray:
    """A copy of n elements at ptr.  One memmove into a fresh array:
    numpy.ctypeslib.as_array would build a new ctypes array and pointer type
    for every call (≈ 0.15 ms each, most of a step's host time)."""
    out = np.empty(max(n, 0), dtype)
    if n > 0:
        ctypes.memmove(out.ctypes.data, ctypes.cast(ptr, ctypes.c_void_p).value, out.nbytes)
    return out


class NativeStepPlan:
    """One step, as arrays (copied out of the scheduler's buffers)."""

    def __init__(self, p: _Plan):
        B, T = p.num_rows, p.num_tokens
        self.req_id = _arr(p.req_id, B, np.int64)
        self.start = _arr(p.start, B, np.int32)
        self.row_tokens = _arr(p.row_tokens, B, np.int32)
        self.is_prefill = _arr(p.is_prefill, B, np.uint8).astype(bool)
        self.table_width = p.table_width
        self.block_tables = _arr(p.block_tables, B * p.table_width, np.int32).reshape(B, p.table_width)
        self.positions = _arr(p.positions, T, np.int32)
        self.query_start_loc = _arr(p.query_start_loc, B + 1, np.int32)
        self.seq_lens = _arr(p.seq_lens, B, np.int32)
        self.swap_out_pairs = _arr(p.swap_out, 2 * p.num_swap_out, np.int32).reshape(-1, 2)
        self.swap_in_pairs = _arr(p.swap_in, 2 * p.num_swap_in, np.int32).reshape(-1, 2)
        self.finished_ids = _arr(p.finished_ids, p.num_finished, np.int64).tolist()
        self.preempted_ids = _arr(p.preempted_ids, p.num_preempted, np.int64).tolist()
        self.num_tokens = T
        self._rows: Optional[List[ScheduledRow]] = None

    @property
    def num_rows(self) -> int:
        return len(self.req_id)

    @property
    def num_prefill(self) -> int:
        return int(self.is_prefill.sum())

    @property
    def num_decode(self) -> int:
        return self.num_rows - self.num_prefill

    @property
    def swap_out(self) -> List[Tuple[int, int]]:
        return [tuple(x) for x in self.swap_out_pairs.tolist()]

    @property
    def swap_in(self) -> List[Tuple[int, int]]:
        return [tuple(x) for x in self.swap_in_pairs.tolist()]

    @property
    def rows(self) -> List[ScheduledRow]:
        """The rows as scheduler.ScheduledRow objects (block tables unpadded)."""
        if self._rows is None:
            self._rows = []
            for i in range(self.num_rows):
                t = self.block_tables[i]
                self._rows.append(ScheduledRow(int(self.req_id[i]), int(self.start[i]), int(self.row_tokens[i]),
                                               bool(self.is_prefill[i]), t[t >= 0].tolist()))
        return self._rows


class _PoolView:
    def __init__(self, fn, s):
        self._fn, self._s = fn, s

    def num_free(self) -> int:
        return int(self._fn(self._s))


class NativeScheduler:
    """scheduler.Scheduler's interface over the native implementation."""

    def __init__(self, config: SchedulerConfig, gpu_order=None):
        self.cfg = config
        self._lib = ops.lib()
        c = _Config(config.block_size, config.num_gpu_blocks, config.num_cpu_blocks, config.max_num_seqs,
                    config.max_num_batched_tokens, config.max_prefill_chunk, float(config.watermark),
                    1 if config.preemption == "swap" else 0)
        order = None
        if gpu_order is not None:
            order = np.ascontiguousarray(np.asarray(gpu_order, dtype=np.int32))
            if order.shape != (config.num_gpu_blocks,):
                raise ValueError("gpu_order must hold num_gpu_blocks ids")
        self._s = self._lib.pkv_sched_create(ctypes.addressof(c), order.ctypes.data if order is not None else None)
        if not self._s:
            raise ValueError("pkv_sched_create: %s" % self._lib.pkv_last_error().decode())
        self.gpu = _PoolView(self._lib.pkv_sched_num_free_gpu, self._s)
        self.cpu = _PoolView(self._lib.pkv_sched_num_free_cpu, self._s)
        self._plan = _Plan()

    def __del__(self):
        s = getattr(self, "_s", None)
        if s:
            self._lib.pkv_sched_destroy(s)
            self._s = None

    def _check(self, status: int, what: str) -> None:
        if status != 0:
            raise ValueError("%s: %s" % (what, self._lib.pkv_last_error().decode()))

    def add_request(self, req_id: int, prompt_len: int, max_new_tokens: int) -> None:
        self._check(self._lib.pkv_sched_add_request(self._s, int(req_id), int(prompt_len), int(max_new_tokens)),
                    "add_request")

    def has_work(self) -> bool:
        return bool(self._lib.pkv_sched_has_work(self._s))

    def schedule(self) -> NativeStepPlan:
        self._check(self._lib.pkv_sched_schedule(self._s, ctypes.addressof(self._plan)), "schedule")
        return NativeStepPlan(self._plan)

    def complete(self, plan: NativeStepPlan) -> None:
        self._check(self._lib.pkv_sched_complete(self._s), "complete")

    def count(self, state: str) -> int:
        return int(self._lib.pkv_sched_count(self._s, ("waiting", "running", "swapped", "finished").index(state)))

    def request_info(self, req_id: int) -> Tuple[int, int, str]:
        """(num_computed, recompute_to, status) of one request."""
        nc, rt, st = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.pkv_sched_request_info(self._s, int(req_id), ctypes.addressof(nc), ctypes.addressof(rt),
                                                     ctypes.addressof(st)), "request_info")
        return nc.value, rt.value, ("waiting", "running", "swapped", "finished")[st.value]
