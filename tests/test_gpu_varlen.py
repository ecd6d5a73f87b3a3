"""GPU parity of the varlen (chunked prefill + decode) step against the
float64 oracle, through the C ABI.  Needs an MI355X and libpagedkv.so."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_97_amd import ops
from paged_kv_cache_97_amd import workloads as W
from gpu_harness import (assert_attn_close, log, oracle_step, run_step, same_bits, to_dev, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.lib()
    return torch.device("cuda:0")


def _check(wl, dev, label, rel_factor=1.0):
    log("[%s] seed %d: B=%d T=%d NB=%d maxL=%d maxq=%d" % (label, wl.seed, wl.num_seqs, wl.num_tokens,
                                                           wl.num_blocks, wl.max_seq_len, wl.max_query_len))
    t = upload(wl, dev)
    slots, out = run_step(wl, t, decode=False)
    r_slots, r_kc, r_vc, r_out = oracle_step(wl, decode=False)
    assert np.array_equal(slots.cpu().numpy(), r_slots), "slot mapping differs"
    assert same_bits(t["key_cache"], r_kc) and same_bits(t["value_cache"], r_vc), "cache contents differ"
    assert_attn_close(out, r_out, wl.spec.dtype, label, rel_factor)
    return t, out


def test_config5_full_size(dev):
    _check(W.generate(5), dev, "config 5")


def _mixed(**kw):
    base = dict(num_decode=6, num_prefill=3, prefill_chunk=70, prefill_ctx=("uniform", 0, 300),
                decode_len=("lognormal", 200.0, W.LOGNORMAL_SIGMA, 16, 600))
    base.update(kw)
    return W.reduced(5, **base)


SMALL = {
    "gqa8-bs16": _mixed(),
    "gqa8-pure-prefill": _mixed(num_decode=0, num_prefill=4, prefill_chunk=33, prefill_ctx=("uniform", 0, 0)),
    "gqa8-long-chunk": _mixed(num_decode=3, num_prefill=2, prefill_chunk=300, prefill_ctx=("uniform", 0, 900)),
    "mha-d128": _mixed(num_q_heads=8, num_kv_heads=8, prefill_chunk=37),
    "gqa4-bs32": _mixed(num_q_heads=16, num_kv_heads=4, block_size=32, prefill_chunk=48),
    "gqa16-d64": _mixed(num_q_heads=32, num_kv_heads=2, head_dim=64, prefill_chunk=21),
    "gqa2-d64-bs32": _mixed(num_q_heads=8, num_kv_heads=4, head_dim=64, block_size=32, prefill_chunk=64),
    "gqa6-odd": _mixed(num_q_heads=12, num_kv_heads=2, prefill_chunk=11),
    "gqa32": _mixed(num_q_heads=64, num_kv_heads=2, prefill_chunk=9),
    # 16 KV heads: two heads in each of the prefill kernel's 8 XCD queues
    "gqa2-kv16": _mixed(num_q_heads=32, num_kv_heads=16, prefill_chunk=45),
    "decode-first": _mixed(prefill_first=False),
    "f32-d64": _mixed(dtype="f32", num_q_heads=4, num_kv_heads=4, head_dim=64, prefill_chunk=40),
    "f32-gqa4-d128": _mixed(dtype="f32", num_q_heads=16, num_kv_heads=4, prefill_chunk=29),
}


@pytest.mark.parametrize("seed", [101, 102])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_reduced_shapes(name, seed, dev):
    _check(W.generate(SMALL[name], seed=seed), dev, name)


@pytest.mark.parametrize("scale", [-1.0 / np.sqrt(128.0), 0.0, 0.75])
@pytest.mark.parametrize("name", ["gqa8-bs16", "gqa8-long-chunk", "gqa4-bs32", "gqa16-d64", "f32-d64"])
def test_any_finite_scale(name, scale, dev):
    """The API takes any finite scale.  A negative one flips which key is
    largest, zero gives uniform weights (the mean of the visible values) and
    a large one makes the running maxima move often; all must match."""
    wl = W.generate(SMALL[name], seed=31)
    wl.scale = float(scale)
    # the relative-L2 self-check grows with the scores (see the decode test)
    _check(wl, dev, "%s scale %g" % (name, scale), max(1.0, abs(scale) * np.sqrt(wl.spec.head_dim)))


@pytest.mark.parametrize("scale", [3.0, 8.0])
@pytest.mark.parametrize("name", ["gqa8-bs16", "gqa8-long-chunk", "gqa4-bs32"])
def test_scores_far_beyond_the_first_chunk(name, scale, dev):
    """Scales so large that later keys' scores exceed a column's early
    maxima by far more than the prefill kernel's rescale slack, many times
    per column: the running references must move exactly."""
    wl = W.generate(SMALL[name], seed=32)
    wl.scale = float(scale)
    _check(wl, dev, "%s scale %g" % (name, scale), max(1.0, abs(scale) * np.sqrt(wl.spec.head_dim)))


def test_more_prefill_sequences_than_the_plan_sorts(dev):
    """600 prefill chunks in one step: past the 512 the plan orders by
    length, the work items follow the batch order instead."""
    spec = _mixed(num_decode=20, num_prefill=600, prefill_chunk=3, prefill_ctx=("uniform", 0, 40))
    _check(W.generate(spec, seed=43), dev, "600 prefills")


def test_mixed_batch_of_the_page_example(dev, golden):
    """Two decode rows plus prefills of 50 and 30 rows: 82 rows, 4 requests."""
    ex = golden["mixed_batch"]
    spec = W.reduced(5, num_q_heads=16, num_kv_heads=4, num_decode=2, num_prefill=2, prefill_chunk=(50, 30),
                     prefill_ctx=("fixed", (0, 0)), decode_len=("fixed", (40, 70)), prefill_first=False)
    wl = W.generate(spec, seed=7)
    assert wl.num_tokens == ex["total_tokens"] and wl.num_seqs == ex["batch_size"]
    assert wl.query_start_loc.tolist() == [0, 1, 2, 52, 82]
    _check(wl, dev, "page-example")


class launches:
    """Mixed varlen calls in one launch (single=True) or through the split +
    merge + prefill launches (the default)."""
    def __init__(self, single: bool):
        self.single = single

    def __enter__(self):
        self.prev = ops.set_varlen_single_launch(self.single)

    def __exit__(self, *exc):
        ops.set_varlen_single_launch(self.prev)


# shapes whose prefill chunks take the workgroup-shared kernel (bf16, head_dim 128)
ONE_LAUNCH = ["decode-first", "gqa32", "gqa4-bs32", "gqa6-odd", "gqa8-bs16", "gqa8-long-chunk",
              "gqa8-pure-prefill", "mha-d128"]


@pytest.mark.parametrize("name", ONE_LAUNCH)
def test_reduced_shapes_one_launch(name, dev):
    """The same steps with prefill chunks and decode rows in one launch."""
    with launches(single=True):
        _check(W.generate(SMALL[name], seed=103), dev, name + " (1 launch)")


def test_config5_full_size_one_launch(dev):
    with launches(single=True):
        _check(W.generate(5), dev, "config 5 (1 launch)")


# decode rows of 1 .. 4,001 tokens (each listed context + the new token): one chunk, a ragged last chunk, ranges on 2 .. 8 waves
DECODE_LENS = (0, 1, 5, 10, 15, 16, 17, 31, 32, 33, 50, 63, 64, 65, 96, 100, 128, 200, 255, 256, 257, 300,
               511, 512, 513, 700, 1000, 1023, 1024, 1025, 1500, 2000, 2047, 2048, 2049, 2500, 3000, 3500,
               3999, 4000)


def _decode_heavy(**kw):
    return _mixed(num_decode=len(DECODE_LENS), num_prefill=2, prefill_chunk=20, prefill_ctx=("uniform", 0, 100),
                  decode_len=("fixed", DECODE_LENS), **kw)


@pytest.mark.parametrize("kw", [dict(), dict(block_size=32), dict(num_q_heads=64, num_kv_heads=2),
                                dict(num_q_heads=40, num_kv_heads=8)], ids=["gqa8", "bs32", "gqa32", "gqa5"])
def test_one_launch_decode_rows(kw, dev):
    """Many decode rows of very different lengths (1 to 4,000 tokens: rows
    of one chunk, and rows split over all 8 waves of a workgroup) queued
    behind two small prefill chunks, with one and with several head tiles,
    in one launch and in three."""
    for single in (True, False):
        with launches(single):
            _check(W.generate(_decode_heavy(**kw), seed=44), dev, "decode-heavy %s single=%d" % (kw, single))


def test_one_launch_is_deterministic_and_leaves_its_counters_zero(dev):
    """Which workgroup runs an item varies from run to run, the results do
    not (every item's split is fixed by its row); the last workgroup resets
    the workspace's counters for the next call."""
    wl = W.generate(_decode_heavy(), seed=45)
    t = upload(wl, dev)
    run_step(wl, t, decode=False)                      # writes the step's K/V
    B, T = wl.num_seqs, wl.num_tokens
    Hq, Hkv, D = wl.spec.num_q_heads, wl.spec.num_kv_heads, wl.spec.head_dim
    nbytes = ops.varlen_workspace_size(B, T, Hq, Hkv, D, wl.max_query_len, wl.spec.block_size, t["query"].dtype)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    outs = []
    with launches(single=True):
        for _ in range(3):
            outs.append(ops.paged_attention_varlen(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                                   t["seq_lens"], t["query_start_loc"], wl.scale, wl.max_query_len,
                                                   wl.max_seq_len, workspace=ws))
            torch.cuda.synchronize()
            assert int(ws[:8].view(torch.int32).abs().sum()) == 0, "counters not reset"
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    assert torch.equal(outs[0].view(torch.int32), outs[2].view(torch.int32))
    r_out = oracle_step(wl, decode=False)[3]
    assert_attn_close(outs[0], r_out, wl.spec.dtype, "deterministic")


def test_shared_workspace_across_calls(dev):
    """Three varlen calls on one workspace: a 16-KV-head step (the prefill
    kernel's per-XCD queues, two heads each), a smaller 8-head step, the
    first again.  Each call rebuilds its item plan and queue counters, so
    the repeated call is bit-identical and both steps match the oracle."""
    wa = W.generate(SMALL["gqa2-kv16"], seed=46)
    wb = W.generate(SMALL["gqa8-long-chunk"], seed=47)
    ta, tb = upload(wa, dev), upload(wb, dev)
    run_step(wa, ta, decode=False)                     # writes each step's K/V
    run_step(wb, tb, decode=False)

    def need(wl, t):
        return ops.varlen_workspace_size(wl.num_seqs, wl.num_tokens, wl.spec.num_q_heads, wl.spec.num_kv_heads,
                                         wl.spec.head_dim, wl.max_query_len, wl.spec.block_size, t["query"].dtype)

    ws = torch.zeros(max(need(wa, ta), need(wb, tb)), dtype=torch.uint8, device=dev)

    def call(wl, t):
        out = ops.paged_attention_varlen(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                         t["seq_lens"], t["query_start_loc"], wl.scale, wl.max_query_len,
                                         wl.max_seq_len, workspace=ws)
        torch.cuda.synchronize()
        return out

    with launches(single=False):
        a1 = call(wa, ta)
        b1 = call(wb, tb)
        a2 = call(wa, ta)
    assert torch.equal(a1.view(torch.int32), a2.view(torch.int32)), "repeated call differs"
    assert_attn_close(a1, oracle_step(wa, decode=False)[3], wa.spec.dtype, "shared workspace, 16 KV heads")
    assert_attn_close(b1, oracle_step(wb, decode=False)[3], wb.spec.dtype, "shared workspace, 8 KV heads")


def test_decode_rows_equal_decode_call_bitwise(dev):
    """With the decode rows in their own launches, they run the decode
    call's kernels on the same split: bit-identical rows."""
    wl = W.generate(SMALL["gqa8-bs16"], seed=21)
    t = upload(wl, dev)
    with launches(single=False):
        _, out = run_step(wl, t, decode=False)
    dec = np.where(~wl.is_prefill)[0]
    rows = torch.from_numpy(wl.query_start_loc[dec].astype(np.int64)).to(dev)
    idx = torch.from_numpy(dec.astype(np.int64)).to(dev)
    ref = ops.paged_attention_decode(t["query"][rows].contiguous(), t["key_cache"], t["value_cache"],
                                     t["block_tables"][idx].contiguous(), t["seq_lens"][idx].contiguous(),
                                     wl.scale, wl.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(out[rows].view(torch.int32), ref.view(torch.int32))


def test_chunked_prefill_equals_one_pass(dev):
    """A 256-token prompt as 4 chunks of 64 (each written before its
    attention) matches one pass over the whole prompt."""
    rng = np.random.default_rng(31)
    N, Hq, Hkv, D, bs = 256, 16, 4, 128, 16
    bits = lambda shape: W._to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    q, k, v = bits((N, Hq, D)), bits((N, Hkv, D)), bits((N, Hkv, D))
    NB = 40
    table = rng.permutation(NB)[: N // bs].astype(np.int32)[None]
    kc = torch.full((NB, bs, Hkv, D), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = kc.clone()
    bt = torch.from_numpy(table).to(dev)
    qd, kd, vd = to_dev(q, "bf16", dev), to_dev(k, "bf16", dev), to_dev(v, "bf16", dev)
    scale = D ** -0.5
    rows = []
    for c in range(4):
        lo, hi = 64 * c, 64 * (c + 1)
        pos = torch.arange(lo, hi, dtype=torch.int32, device=dev)
        qsl = torch.tensor([0, 64], dtype=torch.int32, device=dev)
        sl = ops.compute_slot_mapping(bt, pos, qsl, bs)
        ops.reshape_and_cache(kd[lo:hi].contiguous(), vd[lo:hi].contiguous(), kc, vc, sl)
        rows.append(ops.paged_attention_varlen(qd[lo:hi].contiguous(), kc, vc, bt,
                                               torch.tensor([hi], dtype=torch.int32, device=dev), qsl, scale, 64, hi))
    one = ops.paged_attention_varlen(qd, kc, vc, bt, torch.tensor([N], dtype=torch.int32, device=dev),
                                     torch.tensor([0, N], dtype=torch.int32, device=dev), scale, N, N)
    torch.cuda.synchronize()
    chunked = torch.cat(rows)
    # both against the oracle, and against each other
    kc_h = kc.cpu().view(torch.int16).numpy().view(np.uint16)
    vc_h = vc.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.varlen_attention(q, kc_h, vc_h, table, np.array([N]), np.array([0, N]), scale, "bf16")
    assert_attn_close(one, ref, "bf16", "one pass")
    assert_attn_close(chunked, ref, "bf16", "chunked")
    assert (one - chunked).abs().max().item() <= 2e-2


def test_sequence_order_moves_rows(dev):
    wl = W.generate(SMALL["gqa8-bs16"], seed=41)
    t = upload(wl, dev)
    _, out = run_step(wl, t, decode=False)
    order = np.arange(wl.num_seqs)[::-1].copy()
    qlen = wl.query_lens[order]
    qsl2 = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    src = np.concatenate([np.arange(wl.query_start_loc[s], wl.query_start_loc[s + 1]) for s in order])
    src_t = torch.from_numpy(src.astype(np.int64)).to(dev)
    o_t = torch.from_numpy(order.astype(np.int64)).to(dev)
    out2 = ops.paged_attention_varlen(t["query"][src_t].contiguous(), t["key_cache"], t["value_cache"],
                                      t["block_tables"][o_t].contiguous(), t["seq_lens"][o_t].contiguous(),
                                      torch.from_numpy(qsl2).to(dev), wl.scale, wl.max_query_len, wl.max_seq_len)
    torch.cuda.synchronize()
    for i, s in enumerate(order):
        a = out2[qsl2[i]:qsl2[i + 1]]
        b = out[wl.query_start_loc[s]:wl.query_start_loc[s + 1]]
        if wl.is_prefill[s]:
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        else:
            assert (a - b).abs().max().item() <= 2e-2
