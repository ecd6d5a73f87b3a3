"""Benchmark of the paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--no-cpu]

Default: the headline line is workload 3, a decode iteration of the
128-sequence GQA batch (64 query / 8 KV heads, head_dim 128, bf16 KV, 16-token
blocks, lognormal lengths with median 1500 clipped to [16, 8192]): one
pkv_decode_step call -- the split kernel, which also maps and writes the
step's new tokens into their slots, then the merge kernel.  The same JSON
line then carries, under "configs", every other workload timed the same way:
1 (tiny fp32), 2 (MHA bf16), 3 with E4M3 pools, 4 (long contexts with a
shared prefix; logical and unique bytes), 5 (the mixed chunked-prefill +
decode step through write_new_tokens + the varlen call, whose dominant kernel
is the MFMA-bound prefill kernel).  --config N times one workload alone.
--blocks times the copy-on-write block copy and the swap to and from pinned
host memory; --serve the step driver.  Inputs are resident in HBM before
timing starts.

value = KV bytes read per step / mean step time over K back-to-back steps
(GB/s, 1 GB = 1e9 B), where KV bytes = sum(seq_len) * 2 (K and V) *
num_kv_heads * head_dim * element size -- each sequence's K/V read once per
KV head, as GQA grouping allows.  step_ms = each step between its own events.
roofline.achieved = the same bytes / mean duration of the dominant kernel
alone, from HIP events the library records around it on its stream during a
second pass of K steps.
cpu_baseline = the float64 oracle over the whole step on a fork-started pool
of worker processes (BLAS one thread each), before the GPU is touched; its
first pass is also what every GPU row of the step is compared with
(oracle_check).  Other workloads are checked on a sample of sequences.
cold_step_ms = each step timed alone after a streaming read of 1 GiB of other
data; cold_step_after_write_ms after an overwrite of 1 GiB; hbm_stream_read_GBps
= the library's plain streaming read over 4 GiB (pkv_stream_read), the read
rate this part reaches in practice.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
W_BF16_NAN = np.uint16(0x7FC0)                # the workloads' free-slot poison (bf16 NaN)
MFMA_BF16_TFLOPS = 2500.0
METRIC = "paged-attn decode KV GB/s (% of MI355X HBM peak); seq-tokens/s per step"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
# The decode kernels and the host code that sets their split (worker count,
# segment cost, dynamic share): a stored counter record is used only while
# all of these are unchanged.
KERNEL_SOURCES = ["paged_kv_cache_97_amd/csrc/decode_kernels.hip", "paged_kv_cache_97_amd/csrc/decode_segment.h",
                  "paged_kv_cache_97_amd/csrc/common.h",
                  "paged_kv_cache_97_amd/csrc/tiles.h", "paged_kv_cache_97_amd/csrc/launch.h",
                  "paged_kv_cache_97_amd/csrc/api.hip"]
# The same for the prefill kernel's record (the prefill kernel, its item
# plan, the shared tiles and the host code that launches it).
PREFILL_SOURCES = ["paged_kv_cache_97_amd/csrc/prefill_lds_kernels.hip", "paged_kv_cache_97_amd/csrc/prefill_plan.h",
                   "paged_kv_cache_97_amd/csrc/common.h", "paged_kv_cache_97_amd/csrc/tiles.h",
                   "paged_kv_cache_97_amd/csrc/launch.h", "paged_kv_cache_97_amd/csrc/varlen_kernels.hip",
                   "paged_kv_cache_97_amd/csrc/api.hip"]
CALIB_BYTES = 256 << 20
FP8_K_SCALE, FP8_V_SCALE = 0.0125, 0.02      # per-pool scales of the E4M3 runs


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_key(cfg: int, fp8: bool) -> str:
    return "config%d-%s" % (cfg, "fp8" if fp8 else "auto")


def _load_traffic(key: str, prefill: bool = False):
    """Counter-measured HBM bytes per launch of a workload's split kernel (or,
    with prefill, of its prefill kernel), if they were taken on the current
    sources of that kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec:
        return None
    if prefill:
        ok = "prefill_traffic_bytes_per_launch" in rec and \
            rec.get("prefill_source_hash") == kernel_source_hash(PREFILL_SOURCES)
    else:
        ok = rec.get("source_hash") == kernel_source_hash()
    return rec if ok else None


def summarize(fetch_dir: str, write_dir: str, kv_bytes: int, cmd: str) -> dict:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of each kernel, calibrated by
    the same counters on a plain device copy of CALIB_BYTES."""
    import csv
    import glob

    def read(d, counter):
        rows = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                rows += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        return rows

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read(d, counter)
        calib = [float(r["Counter_Value"]) for r in rows
                 if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 65536]
        if not calib:
            raise SystemExit("no calibration copy found in %s" % d)
        factor = (CALIB_BYTES / 1024.0) / (sum(calib) / len(calib))
        per = {}
        for r in rows:
            name = r["Kernel_Name"]
            per.setdefault(name, []).append(float(r["Counter_Value"]))
        out[counter] = {"calibration_factor": factor,
                        "kernels": {k: {"dispatches": len(v), "raw_kib_mean": sum(v) / len(v),
                                        "bytes_per_launch": sum(v) / len(v) * 1024.0 * factor}
                                    for k, v in per.items()}}
    split = [k for k in out["FETCH_SIZE"]["kernels"] if "decode_split" in k]
    rec = {"source_hash": kernel_source_hash(), "command": cmd, "algorithmic_kv_bytes": kv_bytes,
           "counters": out}
    if split:
        fb = out["FETCH_SIZE"]["kernels"][split[0]]["bytes_per_launch"]
        wb = out["WRITE_SIZE"]["kernels"].get(split[0], {}).get("bytes_per_launch", 0.0)
        rec["split_kernel"] = split[0]
        rec["traffic_bytes_per_launch"] = fb + wb
        rec["fetch_bytes_per_launch"] = fb
        rec["write_bytes_per_launch"] = wb
    pre = [k for k in out["FETCH_SIZE"]["kernels"] if "prefill_lds_kernel" in k]
    if pre:
        fb = out["FETCH_SIZE"]["kernels"][pre[0]]["bytes_per_launch"]
        wb = out["WRITE_SIZE"]["kernels"].get(pre[0], {}).get("bytes_per_launch", 0.0)
        rec.update({"prefill_kernel": pre[0], "prefill_source_hash": kernel_source_hash(PREFILL_SOURCES),
                    "prefill_traffic_bytes_per_launch": fb + wb, "prefill_fetch_bytes_per_launch": fb,
                    "prefill_write_bytes_per_launch": wb})
    return rec


def prefill_flops(wl) -> int:
    """Multiply-add flops of the unmasked (query row, key) pairs of prefill
    rows: 2 (QK) + 2 (PV) per head and dim."""
    sp = wl.spec
    total = 0
    for s in np.where(wl.is_prefill)[0]:
        q = int(wl.query_lens[s])
        ctx = int(wl.seq_lens[s]) - q
        total += (q * ctx + q * (q + 1) // 2) * 4 * sp.num_q_heads * sp.head_dim
    return total


def _fp8_sample(oracle, wl, kc, vc, s, scales):
    """E4M3 pools holding only sequence s's blocks (free slots zeroed before
    quantising) and its table renumbered into them."""
    bs = wl.spec.block_size
    nblk = -(-int(wl.seq_lens[s]) // bs)
    ids = [int(b) for b in wl.block_tables[s, :nblk]]
    nan = W_BF16_NAN
    kb = np.where(kc[ids] == nan, 0, kc[ids]).astype(np.uint16)
    vb = np.where(vc[ids] == nan, 0, vc[ids]).astype(np.uint16)
    table = np.full((1, wl.block_tables.shape[1]), -1, np.int32)
    table[0, :nblk] = np.arange(nblk)
    return oracle.quantize_kv(kb, "bf16", scales[0]), oracle.quantize_kv(vb, "bf16", scales[1]), table


# ----------------------------------------------------------------- the CPU leg
# Everything below up to bench_blocks is the benchmark's CPU-baseline leg: the
# only code here that runs the float64 oracle.  It times the oracle on the
# host cores and keeps the rows it computed, which the GPU rows of the same
# step are then compared with.

def _host_info() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"host_cpu_model": model, "host_cpu_count": os.cpu_count(), "host_affinity": affinity}


def _pool_workers() -> int:
    """Worker processes of the oracle pool: every core this process may run
    on, at most 16 -- a one-GPU share of the host (the bench host gives one
    GPU's jobs 16 cores, whatever os.cpu_count() reports)."""
    return max(1, min(16, _host_info()["host_affinity"]))


_POOL = {}                                       # inherited by the forked workers


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_seq_rows(i: int):
    """Oracle rows of sequence i of the step (its decode row, or its chunk's
    rows), from the pools after the step's write."""
    import oracle
    st = _POOL
    r0, r1 = int(st["qsl"][i]), int(st["qsl"][i + 1])
    return oracle.varlen_attention(st["q"][r0:r1], st["kc"], st["vc"], st["bt"][i:i + 1], st["sl"][i:i + 1],
                                   np.array([0, r1 - r0]), st["scale"], st["dtype"])


def cpu_baseline_pool(wl, budget_s: float = 12.0) -> tuple:
    """The oracle's attention for every sequence of the step (after the step's
    cache write), one sequence per task on a fork-started process pool with
    BLAS at one thread per worker, repeated over the batch until about
    budget_s of wall time (at least one pass).  Must run before the GPU is
    initialised (the workers are forked).  Returns (record, the oracle's rows
    of the first pass [T, Hq, D])."""
    import multiprocessing as mp
    import oracle
    slots = oracle.slot_mapping(wl.block_tables, wl.positions, wl.query_start_loc, wl.spec.block_size)
    kc, vc = oracle.reshape_and_cache(wl.key, wl.value, wl.key_cache, wl.value_cache, slots)
    _POOL.update(q=wl.query, kc=kc, vc=vc, bt=wl.block_tables, sl=wl.seq_lens, qsl=wl.query_start_loc,
                 scale=wl.scale, dtype=wl.spec.dtype)
    B = wl.num_seqs
    # one worker: sequences in batch order for about 3 s (the single-core rate)
    t0 = time.perf_counter()
    n1 = r1 = tok1 = 0
    while n1 < B and time.perf_counter() - t0 < 3.0:
        r1 += int(wl.query_lens[n1])
        tok1 += int(wl.seq_lens[n1])
        _oracle_seq_rows(n1)
        n1 += 1
    single = time.perf_counter() - t0
    workers = _pool_workers()
    passes = 0
    with mp.get_context("fork").Pool(workers, initializer=_pool_init) as pool:
        pool.map(_oracle_seq_rows, range(min(B, workers)), chunksize=1)          # start-up, untimed
        t0 = time.perf_counter()
        first = None
        while True:
            res = pool.map(_oracle_seq_rows, range(B), chunksize=1)
            if first is None:
                first = np.concatenate(res)
            passes += 1
            wall = time.perf_counter() - t0
            if wall >= budget_s:
                break
    _POOL.clear()
    sp = wl.spec
    per_tok = 2 * sp.num_kv_heads * sp.head_dim * wl.elem_bytes
    pass_bytes = int(wl.seq_lens.astype(np.int64).sum()) * per_tok
    host = _host_info()
    rec = {"value": round(passes * pass_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
           "sample": "float64 NumPy oracle attention over the whole step (%d sequences, %d query rows, after the "
                     "step's cache write), %d pass%s, one sequence per task on %d worker processes (fork, BLAS "
                     "1 thread each), %.1f s wall" % (B, wl.num_tokens, passes, "" if passes == 1 else "es", workers,
                                                      wall),
           "seq_tokens_per_s": round(passes * wl.num_tokens / wall, 2),
           "single_worker": {"value": round(tok1 * per_tok / single / 1e9, 4), "unit": "GB/s",
                             "seq_tokens_per_s": round(r1 / single, 2), "sequences": n1, "wall_s": round(single, 3)},
           "workers": workers, **host}
    return rec, first


def oracle_sample(wl, seqs, fp8_scales=None) -> tuple:
    """Oracle rows of the given sequences (in-process, one core): decode rows
    for decode workloads, each sequence's rows of the varlen step otherwise.
    Returns (rows [n_rows, Hq, D] float64, the GPU row indices they match,
    wall seconds, query rows, KV tokens)."""
    import oracle
    slots = oracle.slot_mapping(wl.block_tables, wl.positions, wl.query_start_loc, wl.spec.block_size)
    kc, vc = oracle.reshape_and_cache(wl.key, wl.value, wl.key_cache, wl.value_cache, slots)
    outs, rows = [], []
    tokens = 0
    t0 = time.perf_counter()
    for s in seqs:
        r0, r1 = int(wl.query_start_loc[s]), int(wl.query_start_loc[s + 1])
        pk, pv, table, dt = kc, vc, wl.block_tables[s:s + 1], wl.spec.dtype
        q = wl.query[r0:r1]
        if fp8_scales is not None:
            pk, pv, table = _fp8_sample(oracle, wl, kc, vc, s, fp8_scales)
        outs.append(oracle.varlen_attention(q, pk, pv, table, wl.seq_lens[s:s + 1], np.array([0, r1 - r0]),
                                            wl.scale, dt, fp8_scales))
        rows.extend(range(r0, r1))
        tokens += int(wl.seq_lens[s])
    wall = time.perf_counter() - t0
    return np.concatenate(outs), np.array(rows), wall, len(rows), tokens


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    d = got.astype(np.float64) - ref
    n = float(np.linalg.norm(ref))
    return {"max_abs_err": float(np.abs(d).max()) if d.size else 0.0,
            "rel_l2_err": float(np.linalg.norm(d) / n) if n > 0 else float(np.linalg.norm(d)),
            "finite": bool(np.isfinite(got).all())}


def bench_blocks(args) -> int:
    """Block copies at the decode workload's block shape (16 tokens x 8 KV
    heads x 128 dims bf16 = 32 KiB per pool): copy-on-write copies inside a
    GPU pool and a swap-out / swap-in of a batch of blocks through pinned host
    memory.  One JSON line; bytes count reads plus writes of K and V."""
    import torch
    from paged_kv_cache_97_amd import ops
    dev = torch.device("cuda:0")
    bs, Hkv, D = 16, 8, 128
    NB, pairs, NC = 65536, 4096, 8192
    rng = np.random.default_rng(0)
    kc = torch.randn(NB, bs, Hkv, D, device=dev).to(torch.bfloat16)
    vc = torch.randn(NB, bs, Hkv, D, device=dev).to(torch.bfloat16)
    ids = rng.permutation(NB)[:2 * pairs]
    cow = torch.from_numpy(np.stack([ids[:pairs], ids[pairs:]], 1).astype(np.int64)).to(dev)
    hk = torch.empty(NC, bs, Hkv, D, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk).pin_memory()
    out_map = torch.from_numpy(np.stack([ids[:pairs], rng.permutation(NC)[:pairs]], 1).astype(np.int64)).to(dev)
    in_map = torch.from_numpy(np.stack([out_map[:, 1].cpu().numpy(), ids[pairs:]], 1).astype(np.int64)).to(dev)
    blk = bs * Hkv * D * 2
    moved = 2 * pairs * blk                         # K and V blocks per call (each read once, written once)

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_copy = timed(lambda: ops.copy_blocks(kc, vc, cow), args.steps)
    ms_out = timed(lambda: ops.swap_blocks(kc, vc, hk, hv, out_map), max(2, args.steps // 10))
    ms_in = timed(lambda: ops.swap_blocks(hk, hv, kc, vc, in_map), max(2, args.steps // 10))
    # context: torch's own device-to-device copy of the same volume in one
    # contiguous piece (no block gather)
    ref_src = torch.empty(moved // 2, dtype=torch.int16, device=dev).fill_(1)
    ref_dst = torch.empty_like(ref_src)
    ms_ref = timed(lambda: ref_dst.copy_(ref_src), args.steps)
    del ref_src, ref_dst
    print("bench: copy %.4f ms, swap-out %.4f ms, swap-in %.4f ms (%d pairs of 2 x %d B)" % (
        ms_copy, ms_out, ms_in, pairs, blk), file=sys.stderr, flush=True)
    copy_gbs = 2 * moved / (ms_copy * 1e-3) / 1e9
    rec = {
        "metric": "block copy GB/s (HBM read + write) and swap GB/s (PCIe, one direction)",
        "value": round(copy_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_copy, 5), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "cow-copy-4096-blocks-bs16-h8-d128-bf16", "pairs": pairs, "block_bytes": blk,
                   "pool_blocks": NB, "host_blocks": NC},
        "roofline": {"bound": "hbm", "kernel": "block_copy_kernel", "achieved": round(copy_gbs, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(copy_gbs / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": 2 * moved},
        "swap_out_gbs": round(moved / (ms_out * 1e-3) / 1e9, 2),
        "swap_in_gbs": round(moved / (ms_in * 1e-3) / 1e9, 2),
        "swap_out_ms": round(ms_out, 4), "swap_in_ms": round(ms_in, 4),
        "device_copy_gbs": round(2 * moved / (ms_ref * 1e-3) / 1e9, 2),
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_serve(args) -> int:
    """The step driver (scheduler + engine) on the decode workload's model
    shape: 64/8 heads, head_dim 128, 16-token blocks, bf16 (or --kv-cache-dtype
    fp8) pools; 512 requests with lognormal prompts (median 1500 tokens,
    clipped to [16, 8192]) and 32-256 new tokens each, all queued at the start;
    at most 128 running sequences, 2048 batched tokens per step, 512-token
    prefill chunks, a pool of 16384 blocks (262144 tokens).  --warmup steps are
    run untimed, then --steps steps are timed end to end (host scheduling,
    uploads and kernels); one JSON line."""
    import torch
    from paged_kv_cache_97_amd import workloads as W
    from paged_kv_cache_97_amd.engine import Engine
    from paged_kv_cache_97_amd.scheduler import SchedulerConfig
    fp8 = args.kv_cache_dtype == "fp8"
    cfg = SchedulerConfig(block_size=16, num_gpu_blocks=16384, max_num_seqs=128, max_num_batched_tokens=2048,
                          max_prefill_chunk=512, watermark=0.01)
    eng = Engine(cfg, 64, 8, 128, seed=1, kv_cache_dtype="fp8" if fp8 else "bf16",
                 k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE, scheduler=args.scheduler)
    for rid, p, g, _ in W.request_mix(1, 512, prompt=("lognormal", 1500.0, W.LOGNORMAL_SIGMA, 16, 8192),
                                      new_tokens=("uniform", 32, 256)):
        eng.add_request(rid, p, g)
    for _ in range(args.warmup):
        eng.step()
    torch.cuda.synchronize()
    tok = dec = pre_rows = preempt = 0
    host = 0.0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if not eng.has_work():
            break
        h0 = time.perf_counter()
        o = eng.step()
        host += time.perf_counter() - h0
        tok += o.plan.num_tokens
        dec += o.plan.num_decode
        pre_rows += o.plan.num_prefill
        preempt += len(o.plan.preempted_ids)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rec = {
        "metric": "step-driver throughput (tokens processed per second, prefill + decode)",
        "value": round(tok / wall, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / max(1, args.steps), 4), "higher_is_better": True,
        "dtype": "fp8-e4m3 KV, bf16 Q" if fp8 else "bf16", "data": "synthetic",
        "config": {"workload": "serve-512req-lognormal1500-new32to256-h64x8-d128",
                   "max_num_seqs": 128, "max_num_batched_tokens": 2048, "prefill_chunk": 512,
                   "pool_blocks": 16384, "scheduler": args.scheduler},
        "decode_tokens_per_s": round(dec / wall, 1), "prefill_rows": pre_rows, "preemptions": preempt,
        "host_ms_per_step": round(1e3 * host / max(1, args.steps), 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def _sample_seqs(wl, n: int = 8):
    """Sequences whose rows the oracle recomputes for the error check: every
    prefill chunk's sequence (at most two, the longest contexts first) and up
    to n decode sequences spread over the batch, the longest included."""
    pre = [int(s) for s in np.where(wl.is_prefill)[0]]
    pre = sorted(pre, key=lambda s: -int(wl.seq_lens[s]))[:2]
    dec = [int(s) for s in np.where(~wl.is_prefill)[0]]
    pick = set()
    if dec:
        pick.add(max(dec, key=lambda s: int(wl.seq_lens[s])))
        for i in np.linspace(0, len(dec) - 1, num=min(n, len(dec))).astype(int):
            pick.add(dec[int(i)])
    return pre + sorted(pick)[:n]


class GpuCase:
    """One workload resident on the GPU, with its step function."""

    def __init__(self, cfg: int, fp8: bool, two_call: bool, wl=None):
        import torch
        from paged_kv_cache_97_amd import ops
        from paged_kv_cache_97_amd import workloads as W
        self.torch, self.ops = torch, ops
        dev = torch.device("cuda:0")
        self.wl = wl = W.generate(cfg) if wl is None else wl
        self.cfg, self.fp8 = cfg, fp8
        sp = wl.spec
        print("bench: config %d%s (%s) B=%d sum(seq_len)=%d generated" % (
            cfg, " E4M3" if fp8 else "", sp.name, wl.num_seqs, int(wl.seq_lens.sum())), file=sys.stderr, flush=True)

        def up(a):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

        q, key, value = up(wl.query), up(wl.key), up(wl.value)
        kc, vc = up(wl.key_cache), up(wl.value_cache)
        if fp8:
            if sp.dtype != "bf16":
                raise SystemExit("bench.py: --kv-cache-dtype fp8 needs a bf16 workload")
            # E4M3 pools, filled from the resident bf16 pools by the library's
            # own quantising write (every slot; free slots hold garbage codes,
            # as reused blocks would)
            nb_slots = kc.shape[0] * kc.shape[1]
            kc8 = torch.empty(kc.shape, dtype=torch.uint8, device=dev)
            vc8 = torch.empty(vc.shape, dtype=torch.uint8, device=dev)
            ops.reshape_and_cache_fp8(kc.view(nb_slots, sp.num_kv_heads, sp.head_dim),
                                      vc.view(nb_slots, sp.num_kv_heads, sp.head_dim), kc8, vc8,
                                      torch.arange(nb_slots, dtype=torch.int64, device=dev), FP8_K_SCALE,
                                      FP8_V_SCALE)
            torch.cuda.synchronize()
            del kc, vc
            kc, vc = kc8, vc8
        bt, sl, pos, qsl = up(wl.block_tables), up(wl.seq_lens), up(wl.positions), up(wl.query_start_loc)
        slots = torch.empty(wl.num_tokens, dtype=torch.int64, device=dev)
        self.out = out = torch.empty(wl.num_tokens, sp.num_q_heads, sp.head_dim, dtype=torch.float32, device=dev)
        self.varlen = varlen = bool(wl.is_prefill.any())
        ws = torch.zeros(ops.varlen_workspace_size(wl.num_seqs, wl.num_tokens, sp.num_q_heads, sp.num_kv_heads,
                                                   sp.head_dim, wl.max_query_len, sp.block_size, q.dtype),
                         dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        self.fused = fused = not varlen and not two_call
        self.tensors = (q, key, value, kc, vc, bt, sl, pos, qsl, slots, ws)

        # sequences that share a prefix (held once in the pool) are named to
        # the library, which then reads those blocks once per group
        self.shared = shared = bool(sp.shared_prefix_tokens) and fused and not fp8
        groups = torch.tensor([[0, wl.num_seqs, sp.shared_prefix_tokens]], dtype=torch.int32, device=dev)
        if shared:
            ws = torch.zeros(max(ws.numel(), ops.decode_shared_workspace_size(
                wl.num_seqs, sp.num_q_heads, sp.num_kv_heads, sp.head_dim, sp.block_size, q.dtype, 1)),
                dtype=torch.uint8, device=dev)

        def step():
            if shared:
                ops.decode_step_shared(q, key, value, kc, vc, bt, sl, wl.scale, wl.max_seq_len, groups, out=out,
                                       workspace=ws)
                return
            if fused:
                # one call: the new tokens' slot mapping and cache write run
                # inside the decode attention launch
                if fp8:
                    ops.decode_step_fp8(q, key, value, kc, vc, bt, sl, wl.scale, wl.max_seq_len, FP8_K_SCALE,
                                        FP8_V_SCALE, out=out, workspace=ws)
                else:
                    ops.decode_step(q, key, value, kc, vc, bt, sl, wl.scale, wl.max_seq_len, out=out, workspace=ws)
                return
            if fp8:
                ops.write_new_tokens_fp8(bt, pos, qsl, sp.block_size, key, value, kc, vc, FP8_K_SCALE, FP8_V_SCALE,
                                         slots)
                if varlen:
                    ops.paged_attention_varlen_fp8(q, kc, vc, bt, sl, qsl, wl.scale, wl.max_query_len,
                                                   wl.max_seq_len, FP8_K_SCALE, FP8_V_SCALE, out=out, workspace=ws)
                else:
                    ops.paged_attention_decode_fp8(q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, FP8_K_SCALE,
                                                   FP8_V_SCALE, out=out, workspace=ws)
                return
            # slot mapping + cache write of the step's new tokens (one fused kernel)
            ops.write_new_tokens(bt, pos, qsl, sp.block_size, key, value, kc, vc, slots)
            if varlen:
                ops.paged_attention_varlen(q, kc, vc, bt, sl, qsl, wl.scale, wl.max_query_len, wl.max_seq_len,
                                           out=out, workspace=ws)
            else:
                ops.paged_attention_decode(q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, out=out, workspace=ws)

        self.step = step

    # bytes and flops of one step
    def kv_bytes(self) -> int:
        return self.wl.kv_bytes_logical() // (2 if self.fp8 else 1)

    def kv_bytes_unique(self) -> int:
        return self.wl.kv_bytes_unique() // (2 if self.fp8 else 1)

    def step_name(self) -> str:
        f = "_fp8" if self.fp8 else ""
        if self.shared:
            return ("decode_step_shared (slot mapping + reshape_and_cache fused into paged decode attention; the "
                    "%d-token shared prefix read once for all %d sequences)" % (self.wl.spec.shared_prefix_tokens,
                                                                              self.wl.num_seqs))
        if self.fused:
            return "decode_step%s (slot mapping + reshape_and_cache fused into paged decode attention)" % f
        return "write_new_tokens%s (slot mapping + reshape_and_cache) + paged_attention_%s%s" % (
            f, "varlen" if self.varlen else "decode", f)

    def kernel_name(self) -> str:
        if self.varlen:
            return "mixed_varlen_kernel" if self.ops.varlen_single_launch() else "prefill_kernel"
        return "decode_split_kernel"

    def decode_row_kv_bytes(self) -> int:
        """KV bytes the decode rows of a varlen step read."""
        wl, sp = self.wl, self.wl.spec
        esize = 1 if self.fp8 else (4 if sp.dtype == "f32" else 2)
        return int(wl.seq_lens[~wl.is_prefill].sum()) * sp.num_kv_heads * sp.head_dim * 2 * esize

    def warmup(self, n: int):
        for _ in range(n):
            self.step()
        self.torch.cuda.synchronize()

    def time_back_to_back(self, n: int) -> float:
        """Mean ms per step of n whole steps between two stream events, with
        nothing else recorded (the contract's timing)."""
        torch = self.torch
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(n):
            self.step()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    def time_kernel(self, n: int) -> list:
        """Per-launch ms of the dominant kernel (split kernel for decode, prefill
        kernel for varlen), from HIP events the library records on its stream
        right before and after it."""
        ops = self.ops
        evs = [(ops.HipEvent(), ops.HipEvent()) for _ in range(n)]
        self.torch.cuda.synchronize()
        for e0, e1 in evs:
            ops.set_profile_events(e0, e1)
            self.step()
        ops.set_profile_events(None, None)
        self.torch.cuda.synchronize()
        return [ops.HipEvent.elapsed_ms(e0, e1) for e0, e1 in evs]

    def time_each(self, n: int, flush=None) -> list:
        """ms of each step alone: stream events right around it, after an
        optional flush enqueued outside the events."""
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            if flush is not None:
                flush()
            e0.record()
            self.step()
            e1.record()
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in ev]

    def rows(self, idx) -> np.ndarray:
        return self.out[self.torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(self.out.device)].cpu().numpy()


def _dist(ms: list) -> dict:
    return {"median": round(float(np.median(ms)), 5), "min": round(float(np.min(ms)), 5),
            "p90": round(float(np.percentile(ms, 90)), 5), "mean": round(float(np.mean(ms)), 5)}


def _roofline(case: GpuCase, kern_ms: list) -> dict:
    k_mean = float(np.mean(kern_ms))
    if case.varlen:
        flops = prefill_flops(case.wl)
        achieved = flops / (k_mean * 1e-3) / 1e12
        tr = _load_traffic(traffic_key(case.cfg, case.fp8), prefill=True) \
            if case.kernel_name() == "prefill_kernel" else None
        rec = {"bound": "mfma", "kernel": case.kernel_name(), "achieved": round(achieved, 2),
               "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_TFLOPS, 4),
               "traffic": round(tr["prefill_traffic_bytes_per_launch"]) if tr else None,
               "kernel_ms_mean": round(k_mean, 5),
               "kernel_ms_min": round(float(np.min(kern_ms)), 5), "flops_per_launch": flops}
        if case.kernel_name() == "mixed_varlen_kernel":
            # the one launch also runs the decode rows: achieved charges their
            # time to the prefill flops; the serial bound prices both at peak
            dkv = case.decode_row_kv_bytes()
            bound_ms = flops / (MFMA_BF16_TFLOPS * 1e12) * 1e3 + dkv / (HBM_PEAK_GBPS * 1e9) * 1e3
            rec.update({"decode_row_kv_bytes": dkv, "serial_peak_bound_ms": round(bound_ms, 5),
                        "frac_of_serial_peak_bound": round(bound_ms / k_mean, 4)})
        return rec
    kvb = case.kv_bytes()
    achieved = kvb / (k_mean * 1e-3) / 1e9
    tr = None if case.varlen else _load_traffic(traffic_key(case.cfg, case.fp8))
    return {"bound": "hbm", "kernel": case.kernel_name(), "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": round(tr["traffic_bytes_per_launch"]) if tr else None,
            "kernel_ms_mean": round(k_mean, 5), "kernel_ms_min": round(float(np.min(kern_ms)), 5),
            "bytes_per_launch": kvb}


def config_record(case: GpuCase, ms_step: float, each_ms: list, kern_ms: list, check: dict) -> dict:
    """The per-workload summary the suite line carries."""
    wl, sp = case.wl, case.wl.spec
    kvb = case.kv_bytes()
    rec = {"workload": sp.name + (" (E4M3 pools)" if case.fp8 else ""), "seed": wl.seed,
           "num_seqs": wl.num_seqs, "query_rows": wl.num_tokens, "sum_seq_len": int(wl.seq_lens.sum()),
           "kv_cache_dtype": "fp8-e4m3" if case.fp8 else sp.dtype, "step": case.step_name(),
           "ms_per_step": round(ms_step, 5), "step_ms": _dist(each_ms),
           "kv_bytes": kvb, "kv_GBps": round(kvb / (ms_step * 1e-3) / 1e9, 2),
           "pct_of_hbm_peak": round(100.0 * kvb / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
           "seq_tokens_per_s": round(wl.num_tokens / (ms_step * 1e-3), 1),
           "kv_tokens_per_s": round(float(wl.seq_lens.sum()) / (ms_step * 1e-3), 1),
           "roofline": _roofline(case, kern_ms), "oracle_check": check}
    if sp.shared_prefix_tokens:
        u = case.kv_bytes_unique()
        rec["kv_bytes_unique"] = u
        rec["pct_of_hbm_peak_unique"] = round(100.0 * u / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)
        rec["roofline"]["frac_unique"] = round(u / (float(np.mean(kern_ms)) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    if case.varlen:
        rec["decode_rows"] = int((~wl.is_prefill).sum())
        rec["prefill_rows"] = int(wl.query_lens[wl.is_prefill].sum())
        rec["prefill_flops"] = prefill_flops(wl)
        rec["prefill_TFLOPs_at_step"] = round(prefill_flops(wl) / (ms_step * 1e-3) / 1e12, 1)
    return rec


def check_against_oracle(case: GpuCase, ref_rows=None) -> dict:
    """Errors of the GPU rows of the last step against the oracle's rows of the
    same step: the whole batch when ref_rows (the CPU baseline's first pass)
    is given, else a sample of sequences recomputed here."""
    wl = case.wl
    if ref_rows is not None:
        idx = np.arange(wl.num_tokens)
        e = errors(case.rows(idx), ref_rows)
        e.update({"rows": int(len(idx)), "sample": "every row of the step (the CPU baseline's first pass)"})
        return e
    seqs = _sample_seqs(wl)
    ref, idx, wall, nrows, tokens = oracle_sample(wl, seqs, (FP8_K_SCALE, FP8_V_SCALE) if case.fp8 else None)
    e = errors(case.rows(idx), ref)
    e.update({"rows": int(nrows), "sample": "%d sequences (%d query rows, %d KV tokens): %s" % (
        len(seqs), nrows, tokens, ",".join(map(str, seqs))), "oracle_wall_s": round(wall, 3),
        "oracle_cores": 1})
    return e


def bench_case(case: GpuCase, args, ref_rows=None, check=True) -> tuple:
    # The mixed step's MFMA-bound prefill runs about 10 % slower in its first
    # tens of steps on a cold part than afterwards, so it gets at least 20
    # untimed steps.
    case.warmup(max(args.warmup, 20) if case.varlen else args.warmup)
    ms_step = case.time_back_to_back(args.steps)
    kern_ms = case.time_kernel(args.steps)
    each_ms = case.time_each(args.steps)
    chk = check_against_oracle(case, ref_rows) if check else None
    print("bench: %.4f ms/step, %s mean %.4f ms (min %.4f, p90 %.4f)" % (
        ms_step, case.kernel_name(), float(np.mean(kern_ms)), float(np.min(kern_ms)),
        float(np.percentile(kern_ms, 90))), file=sys.stderr, flush=True)
    return ms_step, kern_ms, each_ms, chk


SUITE = [("1", 1, False), ("2", 2, False), ("3-e4m3", 3, True), ("4", 4, False), ("5", 5, False)]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=None,
                    help="run only this workload (default: workload 3 as the headline, then the others)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and the oracle checks")
    ap.add_argument("--kernels-only", action="store_true",
                    help="run warmup + steps untimed, then one plain %d MiB device copy (counter runs)" % (CALIB_BYTES >> 20))
    ap.add_argument("--summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of --kernels-only into %s" % os.path.relpath(TRAFFIC_FILE, ROOT))
    ap.add_argument("--command", default="", help="command line recorded with --summarize")
    ap.add_argument("--kv-cache-dtype", choices=["auto", "fp8"], default="auto",
                    help="auto: pools in the workload's dtype; fp8: OCP E4M3 pools (k/v scales %g/%g)" % (0.0125, 0.02))
    ap.add_argument("--serve", action="store_true",
                    help="run the continuous-batching step driver over a synthetic request stream instead")
    ap.add_argument("--scheduler", choices=["native", "python"], default="native",
                    help="--serve: the native (C++) scheduler or the Python one it mirrors")
    ap.add_argument("--two-call", action="store_true",
                    help="decode: time write_new_tokens + paged_attention_decode instead of the one-call decode_step")
    ap.add_argument("--blocks", action="store_true",
                    help="time the copy-on-write block copy and the GPU <-> pinned host swap instead")
    args = ap.parse_args()
    if args.summarize:
        from paged_kv_cache_97_amd import workloads as W
        cfg = args.config or 3
        fp8 = args.kv_cache_dtype == "fp8"
        wl = W.generate(cfg)
        rec = summarize(args.summarize[0], args.summarize[1], wl.kv_bytes_logical() // (2 if fp8 else 1), args.command)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        try:
            with open(TRAFFIC_FILE) as f:
                allrec = json.load(f)
        except (OSError, ValueError):
            allrec = {}
        allrec[traffic_key(cfg, fp8)] = rec
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(allrec, f, indent=1)
        print(json.dumps({k: v for k, v in rec.items() if k != "counters"}))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: the hot path runs on a single MI355X and this build has "
              "no multi-GPU path (requested --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    from paged_kv_cache_97_amd import workloads as W

    suite = args.config is None
    cfg = 3 if suite else args.config
    fp8 = args.kv_cache_dtype == "fp8"
    wl = W.generate(cfg)
    # The CPU baseline forks its worker pool, so it runs before anything
    # touches the GPU; its first pass is the oracle's answer for every row.
    cpu, ref_rows = None, None
    if not args.no_cpu and not args.kernels_only and not fp8:
        cpu, ref_rows = cpu_baseline_pool(wl)
        print("bench: CPU oracle baseline %.3f GB/s on %d workers" % (cpu["value"], cpu["cores"]),
              file=sys.stderr, flush=True)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from paged_kv_cache_97_amd import ops
    ops.lib()
    if args.blocks:
        return bench_blocks(args)
    if args.serve:
        return bench_serve(args)
    dev = torch.device("cuda:0")
    case = GpuCase(cfg, fp8, args.two_call, wl)
    if args.kernels_only:
        case.warmup(args.warmup)
        for _ in range(args.steps):
            case.step()
        a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        a.fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print("bench: kernels-only pass done (%d steps, calibration copy %d bytes)" % (args.steps, CALIB_BYTES),
              file=sys.stderr, flush=True)
        return 0

    ms_step, kern_ms, each_ms, chk = bench_case(case, args, ref_rows, check=not args.no_cpu)
    # Each step alone after the library's streaming read of 1 GiB of other
    # data (read-only, so no dirty lines are left to write back), and after
    # an overwrite of 1 GiB (plain stores; the step then also pays for the
    # write-back of what the overwrite left dirty in the caches).
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    cold_ms = case.time_each(args.steps, lambda: ops.stream_read(scratch, sink))
    cold_w_ms = case.time_each(args.steps, lambda: scratch.fill_(7))
    del scratch
    # The same streaming read over 4 GiB: the HBM read rate this part reaches
    # in practice, next to the 8 TB/s peak.
    big = torch.ones(1 << 30, dtype=torch.int32, device=dev)
    ops.stream_read(big, sink)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(10):
        ops.stream_read(big, sink)
    r1.record()
    torch.cuda.synchronize()
    stream_gbps = 10 * big.numel() * 4 / (r0.elapsed_time(r1) * 1e-3) / 1e9
    del big
    head = config_record(case, ms_step, each_ms, kern_ms, chk)
    kv_bytes = case.kv_bytes()
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    sp = wl.spec

    def cold(ms, how):
        return {**{k: v for k, v in _dist(ms).items() if k != "mean"},
                "value_at_median": round(kv_bytes / (float(np.median(ms)) * 1e-3) / 1e9, 2),
                "pct_at_median": round(100.0 * kv_bytes / (float(np.median(ms)) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                "how": how}

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8-e4m3 KV, bf16 Q" if fp8 else ("bf16" if sp.dtype == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": sp.name, "num_seqs": wl.num_seqs, "num_q_heads": sp.num_q_heads,
                   "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim, "block_size": sp.block_size,
                   "sum_seq_len": int(wl.seq_lens.sum()), "max_seq_len": wl.max_seq_len, "seed": wl.seed,
                   "kv_cache_dtype": "fp8 (E4M3, k/v scales %g/%g)" % (FP8_K_SCALE, FP8_V_SCALE) if fp8
                   else sp.dtype, "step": case.step_name()},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "seq_tokens_per_s": round(wl.num_tokens / (ms_step * 1e-3), 1),
        "kv_tokens_per_s": round(float(wl.seq_lens.sum()) / (ms_step * 1e-3), 1),
        "step_ms": _dist(each_ms),
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "oracle_check": chk,
        "cold_step_ms": cold(cold_ms, "each step alone, after a streaming read of 1 GiB of other data"),
        "cold_step_after_write_ms": cold(cold_w_ms, "each step alone, after 1 GiB of other data was overwritten "
                                                    "with plain stores"),
        "hbm_stream_read_GBps": round(stream_gbps, 1),
    }
    if suite:
        del case
        torch.cuda.empty_cache()
        cfgs = {"3": head}
        for key, c, f8 in SUITE:
            other = GpuCase(c, f8, False, wl if (c == 3) else None)
            o_ms, o_kern, o_each, o_chk = bench_case(other, args, None, check=not args.no_cpu)
            cfgs[key] = config_record(other, o_ms, o_each, o_kern, o_chk)
            del other
            torch.cuda.empty_cache()
        rec["configs"] = cfgs
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
