"""Benchmark of the paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--no-cpu]

A step is one decode iteration of the 128-sequence GQA workload (64 query /
8 KV heads, head_dim 128, bf16 KV, 16-token blocks, lognormal lengths with
median 1500 clipped to [16, 8192]): one pkv_decode_step call -- the split
kernel, which also maps and writes the step's new tokens into their slots,
then the merge kernel (--two-call: pkv_write_new_tokens, then
pkv_paged_attention_decode).
Inputs are resident in HBM before timing starts.  Prints one JSON line.
--config N runs another seeded workload the same way (1-4 decode; 5 is the
mixed chunked-prefill + decode step, timed through the varlen call, whose
dominant kernel is the MFMA-bound prefill kernel).  --blocks times the
copy-on-write block copy and the swap to and from pinned host memory.

value = KV bytes read per step / step time (GB/s, 1 GB = 1e9 B), where KV
bytes = sum(seq_len) * 2 (K and V) * num_kv_heads * head_dim * 2 B -- each
sequence's K/V read once per KV head, as GQA grouping allows.
roofline.achieved = the same bytes / mean duration of the split kernel alone,
from HIP events the library records around that kernel on its stream during a
second pass of the same K steps (the events are kept out of the first, timed
pass because each record adds a few microseconds of queue serialisation).
cpu_baseline = the float64 oracle on a bounded sample of the same batch.
cold_step_ms = the same step timed alone after 1 GiB of scratch was written
(no cache holds the previous step's data); hbm_stream_read_GBps = the
library's plain streaming read over 4 GiB (pkv_stream_read), the read rate
this part reaches in practice.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_kernel_traffic.json")
KERNEL_SOURCES = ["paged_kv_cache_97_amd/csrc/decode_kernels.hip", "paged_kv_cache_97_amd/csrc/common.h",
                  "paged_kv_cache_97_amd/csrc/tiles.h", "paged_kv_cache_97_amd/csrc/launch.h"]
CALIB_BYTES = 256 << 20
FP8_K_SCALE, FP8_V_SCALE = 0.0125, 0.02      # per-pool scales of the E4M3 runs


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _load_traffic():
    """Counter-measured HBM bytes per launch of the split kernel, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec


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
    split = [k for k in out["FETCH_SIZE"]["kernels"] if "decode_split_kernel" in k]
    rec = {"source_hash": kernel_source_hash(), "command": cmd, "algorithmic_kv_bytes": kv_bytes,
           "counters": out}
    if split:
        fb = out["FETCH_SIZE"]["kernels"][split[0]]["bytes_per_launch"]
        wb = out["WRITE_SIZE"]["kernels"].get(split[0], {}).get("bytes_per_launch", 0.0)
        rec["split_kernel"] = split[0]
        rec["traffic_bytes_per_launch"] = fb + wb
        rec["fetch_bytes_per_launch"] = fb
        rec["write_bytes_per_launch"] = wb
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


def _cpu_baseline(wl, budget_s: float = 12.0, fp8_scales=None):
    """Time the oracle's attention on the batch's sequences, one at a time in
    batch order (wrapping round to the first sequence after the last), until
    about budget_s of work is done; report the KV GB/s of that sample (the
    same bytes model as the GPU value).  With fp8_scales the oracle reads E4M3
    pools (quantised per sequence outside the timed part)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    slots = oracle.slot_mapping(wl.block_tables, wl.positions, wl.query_start_loc, wl.spec.block_size)
    kc, vc = oracle.reshape_and_cache(wl.key, wl.value, wl.key_cache, wl.value_cache, slots)
    decode = not wl.is_prefill.any()
    dt = 0.0
    done, tokens, rows = 0, 0, 0
    while dt < budget_s:
        i = done % wl.num_seqs
        s = slice(i, i + 1)
        r0, r1 = int(wl.query_start_loc[i]), int(wl.query_start_loc[i + 1])
        pk, pv, table, dts = kc, vc, wl.block_tables[s], wl.spec.dtype
        if fp8_scales is not None:
            pk, pv, table = _fp8_sample(oracle, wl, kc, vc, i, fp8_scales)
        t0 = time.perf_counter()
        if decode:
            oracle.decode_attention(wl.query[r0:r1], pk, pv, table, wl.seq_lens[s], wl.scale, dts, fp8_scales)
        else:
            oracle.varlen_attention(wl.query[r0:r1], pk, pv, table, wl.seq_lens[s], np.array([0, r1 - r0]),
                                    wl.scale, dts, fp8_scales)
        dt += time.perf_counter() - t0
        tokens += int(wl.seq_lens[i])
        rows += r1 - r0
        done += 1
    sp = wl.spec
    nbytes = tokens * 2 * sp.num_kv_heads * sp.head_dim * (1 if fp8_scales is not None else wl.elem_bytes)
    passes, extra = divmod(done, wl.num_seqs)
    covered = ("%d full pass%s over the %d sequences%s" % (passes, "" if passes == 1 else "es", wl.num_seqs,
                                                          " plus the first %d" % extra if extra else "")
               if passes else "the first %d of %d sequences" % (done, wl.num_seqs))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": "float64 NumPy oracle %s%s attention, %s (%d query rows, %d KV tokens), %.1f s"
                      % ("E4M3 " if fp8_scales else "", "decode" if decode else "varlen", covered, rows, tokens, dt),
            "seq_tokens_per_s": round(rows / dt, 3)}


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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
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
        wl = W.generate(args.config)
        rec = summarize(args.summarize[0], args.summarize[1], wl.kv_bytes_logical(), args.command)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps({k: v for k, v in rec.items() if k != "counters"}))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: the hot path runs on a single MI355X and this build has "
              "no multi-GPU path (requested --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    from paged_kv_cache_97_amd import ops
    from paged_kv_cache_97_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.blocks:
        return bench_blocks(args)
    if args.serve:
        return bench_serve(args)
    dev = torch.device("cuda:0")
    ops.lib()
    wl = W.generate(args.config)
    sp = wl.spec
    print("bench: config %d (%s) B=%d sum(seq_len)=%d generated" % (args.config, sp.name, wl.num_seqs,
          int(wl.seq_lens.sum())), file=sys.stderr, flush=True)

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    q, key, value = up(wl.query), up(wl.key), up(wl.value)
    kc, vc = up(wl.key_cache), up(wl.value_cache)
    fp8 = args.kv_cache_dtype == "fp8"
    if fp8:
        if sp.dtype != "bf16":
            print("bench.py: --kv-cache-dtype fp8 needs a bf16 workload", file=sys.stderr)
            return 2
        # E4M3 pools, filled from the resident bf16 pools by the library's own
        # quantising write (every slot; free slots hold garbage codes, as reused
        # blocks would)
        nb_slots = kc.shape[0] * kc.shape[1]
        kc8 = torch.empty(kc.shape, dtype=torch.uint8, device=dev)
        vc8 = torch.empty(vc.shape, dtype=torch.uint8, device=dev)
        ops.reshape_and_cache_fp8(kc.view(nb_slots, sp.num_kv_heads, sp.head_dim),
                                  vc.view(nb_slots, sp.num_kv_heads, sp.head_dim), kc8, vc8,
                                  torch.arange(nb_slots, dtype=torch.int64, device=dev), FP8_K_SCALE, FP8_V_SCALE)
        torch.cuda.synchronize()
        del kc, vc
        kc, vc = kc8, vc8
    bt, sl, pos, qsl = up(wl.block_tables), up(wl.seq_lens), up(wl.positions), up(wl.query_start_loc)
    slots = torch.empty(wl.num_tokens, dtype=torch.int64, device=dev)
    out = torch.empty(wl.num_tokens, sp.num_q_heads, sp.head_dim, dtype=torch.float32, device=dev)
    varlen = bool(wl.is_prefill.any())
    ws = torch.empty(ops.varlen_workspace_size(wl.num_seqs, wl.num_tokens, sp.num_q_heads, sp.num_kv_heads,
                                               sp.head_dim, wl.max_query_len, sp.block_size, q.dtype),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    fused = not varlen and not args.two_call

    def step():
        if fused:
            # one call: the new tokens' slot mapping and cache write run inside
            # the decode attention launch
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
                ops.paged_attention_varlen_fp8(q, kc, vc, bt, sl, qsl, wl.scale, wl.max_query_len, wl.max_seq_len,
                                               FP8_K_SCALE, FP8_V_SCALE, out=out, workspace=ws)
            else:
                ops.paged_attention_decode_fp8(q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, FP8_K_SCALE, FP8_V_SCALE,
                                               out=out, workspace=ws)
            return
        # slot mapping + cache write of the step's new tokens (one fused kernel)
        ops.write_new_tokens(bt, pos, qsl, sp.block_size, key, value, kc, vc, slots)
        if varlen:
            ops.paged_attention_varlen(q, kc, vc, bt, sl, qsl, wl.scale, wl.max_query_len, wl.max_seq_len,
                                       out=out, workspace=ws)
        else:
            ops.paged_attention_decode(q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.kernels_only:
        for _ in range(args.steps):
            step()
        a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        a.fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print("bench: kernels-only pass done (%d steps, calibration copy %d bytes)" % (args.steps, CALIB_BYTES),
              file=sys.stderr, flush=True)
        return 0

    # Region A (the contract): K whole steps between two stream events, with
    # nothing else recorded, so the step time carries no profiling markers.
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_stop.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_stop)
    # Region B: the same K steps again, now with HIP events that the library
    # records on its stream right before and after the dominant kernel (split
    # kernel for decode, prefill kernel for varlen), giving its duration per
    # launch.
    evs = [(ops.HipEvent(), ops.HipEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        ops.set_profile_events(e0, e1)
        step()
    ops.set_profile_events(None, None)
    torch.cuda.synchronize()
    kern_ms = [ops.HipEvent.elapsed_ms(e0, e1) for e0, e1 in evs]
    ms_step = total_ms / args.steps
    # Region C: each step timed alone after the library's streaming read of
    # 1 GiB of other data (outside its events, read-only so no dirty lines
    # are left to write back), so neither the L2s nor the 256 MB last-level
    # cache hold anything of the previous step.
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    cold = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in cold:
        ops.stream_read(scratch, sink)
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    cold_ms = [e0.elapsed_time(e1) for e0, e1 in cold]
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
    kv_bytes = wl.kv_bytes_logical() // (2 if fp8 else 1)
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    k_mean = float(np.mean(kern_ms))
    kname = "prefill_kernel" if varlen else "decode_split_kernel"
    print("bench: %.4f ms/step, %s mean %.4f ms (min %.4f, p90 %.4f)" % (
        ms_step, kname, k_mean, float(np.min(kern_ms)), float(np.percentile(kern_ms, 90))),
        file=sys.stderr, flush=True)
    if varlen:
        flops = prefill_flops(wl)
        achieved = flops / (k_mean * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 2), "peak": MFMA_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_TFLOPS, 4), "traffic": None,
                "kernel_ms_mean": round(k_mean, 5), "kernel_ms_min": round(float(np.min(kern_ms)), 5),
                "flops_per_launch": flops}
    else:
        achieved = kv_bytes / (k_mean * 1e-3) / 1e9
        tr = _load_traffic() if args.config == 3 and not fp8 else None
        roof = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": round(tr["traffic_bytes_per_launch"]) if tr else None,
                "kernel_ms_mean": round(k_mean, 5), "kernel_ms_min": round(float(np.min(kern_ms)), 5),
                "bytes_per_launch": kv_bytes}
    cpu = None
    if not args.no_cpu:
        cpu = _cpu_baseline(wl, fp8_scales=(FP8_K_SCALE, FP8_V_SCALE) if fp8 else None)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8-e4m3 KV, bf16 Q" if fp8 else ("bf16" if sp.dtype == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": sp.name, "num_seqs": wl.num_seqs, "num_q_heads": sp.num_q_heads,
                   "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim, "block_size": sp.block_size,
                   "sum_seq_len": int(wl.seq_lens.sum()), "max_seq_len": wl.max_seq_len, "seed": wl.seed,
                   "kv_cache_dtype": "fp8 (E4M3, k/v scales %g/%g)" % (FP8_K_SCALE, FP8_V_SCALE) if fp8
                   else sp.dtype,
                   "step": ("decode_step%s (slot mapping + reshape_and_cache fused into paged decode attention)"
                            % ("_fp8" if fp8 else "")) if fused else
                           ("write_new_tokens%s (slot mapping + reshape_and_cache) + paged_attention_%s%s"
                            % ("_fp8" if fp8 else "", "varlen" if varlen else "decode", "_fp8" if fp8 else ""))},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "seq_tokens_per_s": round(wl.num_tokens / (ms_step * 1e-3), 1),
        "kv_tokens_per_s": round(float(wl.seq_lens.sum()) / (ms_step * 1e-3), 1),
        "roofline": roof,
        "cpu_baseline": cpu,
        "cold_step_ms": {"median": round(float(np.median(cold_ms)), 5), "min": round(float(np.min(cold_ms)), 5),
                         "p90": round(float(np.percentile(cold_ms, 90)), 5),
                         "value_at_median": round(kv_bytes / (float(np.median(cold_ms)) * 1e-3) / 1e9, 2),
                         "how": "each step alone, after a streaming read of 1 GiB of other data (caches cold)"},
        "hbm_stream_read_GBps": round(stream_gbps, 1),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
