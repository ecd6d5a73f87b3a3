"""GPU step driver: multi-step continuous-batching runs through the C ABI
(swaps, cache writes, decode/varlen attention) checked at every step against
attention over each request's own tokens, and the written cache slots
against the oracle's encoding of the same rows.  Needs an MI355X and libpagedkv.so."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_97_amd import workloads as W
from paged_kv_cache_97_amd.engine import Engine
from paged_kv_cache_97_amd.scheduler import SchedulerConfig
from gpu_harness import assert_attn_close, log
from serving_harness import dense_rows, step_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("mode,kv", [("recompute", "bf16"), ("swap", "bf16"), ("recompute", "fp8"),
                                     ("swap", "fp8")])
def test_engine_matches_dense_attention_and_written_slots_every_step(mode, kv, dev):
    cfg = SchedulerConfig(block_size=16, num_gpu_blocks=96, num_cpu_blocks=128 if mode == "swap" else 0,
                          max_num_seqs=12, max_num_batched_tokens=640, max_prefill_chunk=256, watermark=0.05,
                          preemption=mode)
    order = np.random.default_rng(17).permutation(96)
    kw = dict(num_q_heads=16, num_kv_heads=2, head_dim=128, seed=9, kv_cache_dtype=kv, gpu_order=order)
    eng = Engine(cfg, device=dev, **kw)
    for rid, p, g, _ in W.request_mix(23, 14, prompt=("lognormal", 200.0, W.LOGNORMAL_SIGMA, 8, 700),
                                      new_tokens=("uniform", 4, 48)):
        eng.add_request(rid, p, g)
    steps, preempted, swapped = 0, 0, 0
    while eng.has_work():
        o = eng.step()
        steps += 1
        preempted += len(o.plan.preempted_ids)
        swapped += len(o.plan.swap_out)
        if not o.plan.rows:
            continue
        torch.cuda.synchronize()
        expect = dense_rows(eng, o.plan)
        assert_attn_close(o.out, expect, "bf16", "step %d (%d rows)" % (steps, len(o.plan.rows)))
        # written slots hold what the oracle's write puts there
        bt, pos, qsl, sl, q, k, v = step_inputs(eng, o.plan)
        slots = oracle.slot_mapping(bt, pos, qsl, cfg.block_size, cfg.num_gpu_blocks)
        blk = torch.from_numpy(slots // cfg.block_size).to(dev)
        off = torch.from_numpy(slots % cfg.block_size).to(dev)
        if kv == "fp8":
            rk, rv = oracle.quantize_kv(k, "bf16", eng.k_scale), oracle.quantize_kv(v, "bf16", eng.v_scale)
            gk = eng.key_cache[blk, off].cpu().numpy()
            gv = eng.value_cache[blk, off].cpu().numpy()
        else:
            rk, rv = k, v
            gk = eng.key_cache[blk, off].view(torch.int16).cpu().numpy().view(np.uint16)
            gv = eng.value_cache[blk, off].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
        assert steps < 2000
    log("  %s/%s: %d steps, %d preemptions, %d blocks swapped out" % (mode, kv, steps, preempted, swapped))
    assert preempted > 0
    if mode == "swap":
        assert swapped > 0
    assert eng.sched.gpu.num_free() == cfg.num_gpu_blocks
