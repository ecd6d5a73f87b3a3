"""GPU parity of the one-call decode step (the new token's cache write fused
into the decode attention launch), through the C ABI: bit for bit equal to
the two calls it replaces (write_new_tokens, then paged_attention_decode)
for every tile type, split of the work and edge case, and equal to the
float64 oracle's slot mapping, cache write and attention.  Needs an MI355X
and libpagedkv.so."""
import numpy as np
import pytest
import torch

from paged_kv_cache_97_amd import ops
from paged_kv_cache_97_amd import workloads as W
from gpu_harness import (K_SCALE, V_SCALE, assert_attn_close, log, oracle_fp8_step, oracle_step, same_bits, upload,
                         upload_fp8)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.lib()
    return torch.device("cuda:0")


SHAPES = {
    "gqa8-bs16": W.reduced(3, num_decode=24, decode_len=("lognormal", 300.0, W.LOGNORMAL_SIGMA, 1, 1500)),
    "mha-bf16": W.reduced(2, num_decode=8, decode_len=("uniform", 1, 700)),
    "gqa4-bs32": W.reduced(4, num_decode=4, decode_len=("uniform", 2100, 4000)),
    "gqa16-d64": W.reduced(3, num_decode=10, num_q_heads=32, num_kv_heads=2, head_dim=64,
                           decode_len=("uniform", 1, 900)),
    "gqa32-d128-bs32": W.reduced(3, num_decode=6, num_q_heads=64, num_kv_heads=2, block_size=32,
                                 decode_len=("uniform", 30, 700)),
    "gqa2-d64-bs32": W.reduced(3, num_decode=9, num_q_heads=8, num_kv_heads=4, head_dim=64, block_size=32,
                               decode_len=("uniform", 1, 400)),
    "gqa6-odd": W.reduced(3, num_decode=7, num_q_heads=12, num_kv_heads=2, decode_len=("uniform", 1, 300)),
    "f32-d128": W.reduced(1, num_decode=6, num_q_heads=8, num_kv_heads=2, head_dim=128, pool_blocks=None,
                          decode_len=("uniform", 1, 300), decode_len_is_ctx=False),
    "f32-gqa4-bs32": W.reduced(1, num_decode=5, num_q_heads=16, num_kv_heads=4, block_size=32, pool_blocks=None,
                               decode_len=("uniform", 1, 500), decode_len_is_ctx=False),
    "edges": W.reduced(3, num_decode=12, decode_len=("fixed", (1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 1000))),
}


def _pools(wl, dev, fp8):
    return upload_fp8(wl, dev) if fp8 else upload(wl, dev)


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.uint8)


def _two_calls(wl, t, fp8, seq_lens, positions):
    bs = wl.spec.block_size
    if fp8:
        ops.write_new_tokens_fp8(t["block_tables"], positions, t["query_start_loc"], bs, t["key"], t["value"],
                                 t["key_cache"], t["value_cache"], K_SCALE, V_SCALE)
        return ops.paged_attention_decode_fp8(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                              seq_lens, wl.scale, wl.max_seq_len, K_SCALE, V_SCALE)
    ops.write_new_tokens(t["block_tables"], positions, t["query_start_loc"], bs, t["key"], t["value"],
                         t["key_cache"], t["value_cache"])
    return ops.paged_attention_decode(t["query"], t["key_cache"], t["value_cache"], t["block_tables"], seq_lens,
                                      wl.scale, wl.max_seq_len)


def _one_call(wl, t, fp8, seq_lens):
    if fp8:
        return ops.decode_step_fp8(t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"],
                                   t["block_tables"], seq_lens, wl.scale, wl.max_seq_len, K_SCALE, V_SCALE)
    return ops.decode_step(t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"], t["block_tables"],
                           seq_lens, wl.scale, wl.max_seq_len)


def _compare(wl, dev, fp8, label, edit=None):
    """Run both paths from identical pools; outputs and pools must match bit
    for bit.  edit(t) may change block tables / seq_lens first (host-side)."""
    log("[step %s%s] seed %d B=%d maxL=%d" % (label, " fp8" if fp8 else "", wl.seed, wl.num_seqs, wl.max_seq_len))
    assert not wl.is_prefill.any() and np.array_equal(wl.positions, wl.seq_lens - 1)
    a = _pools(wl, dev, fp8)
    if edit is not None:
        edit(a)
    b = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in a.items()}
    seq_lens = a["seq_lens"]
    positions = seq_lens - 1
    out_a = _two_calls(wl, a, fp8, seq_lens, positions)
    out_b = _one_call(wl, b, fp8, seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out_a), _bits(out_b)), "outputs differ from write + decode"
    assert torch.equal(_bits(a["key_cache"]), _bits(b["key_cache"])), "K pools differ"
    assert torch.equal(_bits(a["value_cache"]), _bits(b["value_cache"])), "V pools differ"
    return b, out_b


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("name", sorted(SHAPES))
def test_step_equals_write_then_decode_bitwise(name, fp8, dev):
    spec = SHAPES[name]
    if fp8 and spec.dtype != "bf16":
        pytest.skip("E4M3 pools take bfloat16 rows")
    _compare(W.generate(spec, seed=301), dev, fp8, name)


@pytest.mark.parametrize("cost", [0, 7])
def test_step_segment_costs_bitwise(cost, dev):
    prev = ops.set_decode_segment_cost(cost)
    try:
        _compare(W.generate(SHAPES["gqa8-bs16"], seed=309), dev, False, "cost=%d" % cost)
        _compare(W.generate(SHAPES["edges"], seed=310), dev, True, "cost=%d" % cost)
    finally:
        ops.set_decode_segment_cost(prev)


@pytest.mark.parametrize("workers", [1, 2, 3, 7, 64, 333, 4096])
def test_step_forced_split_points_bitwise(workers, dev):
    """Every way the split can cut the last chunk off (single-chunk ranges,
    two and three chunks left, whole pairs) keeps both paths identical."""
    prev = ops.set_decode_workers(workers)
    try:
        _compare(W.generate(SHAPES["gqa8-bs16"], seed=302), dev, False, "workers=%d" % workers)
        _compare(W.generate(SHAPES["gqa8-bs16"], seed=303), dev, True, "workers=%d" % workers)
        _compare(W.generate(SHAPES["f32-d128"], seed=304), dev, False, "workers=%d" % workers)
        _compare(W.generate(SHAPES["gqa32-d128-bs32"], seed=305), dev, False, "workers=%d" % workers)
    finally:
        ops.set_decode_workers(prev)


@pytest.mark.parametrize("fp8", [False, True])
def test_step_degenerate_rows_bitwise(fp8, dev):
    """Rows the fused write must leave alone, exactly as the separate write
    does: an empty sequence, a length past the table (clamped attention, no
    write), a last block id of -1 and one past the pool (no write, the pool
    read as the separate path reads it)."""
    wl = W.generate(SHAPES["gqa8-bs16"], seed=306)
    M, bs, NB = wl.block_tables.shape[1], wl.spec.block_size, wl.num_blocks

    def edit(t):
        sl = t["seq_lens"]
        bt = t["block_tables"]
        sl[2] = 0
        sl[4] = M * bs + 7
        for s, bad in ((6, -1), (8, NB), (9, NB + 1000)):
            L = int(sl[s])
            bt[s, (L - 1) // bs] = bad
    b, out = _compare(wl, dev, fp8, "degenerate", edit)
    assert torch.count_nonzero(out[2]) == 0


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_step_matches_oracle_full_size(cfg, dev):
    """The decode workloads as the benchmark runs them (the tiny fp32 pair,
    32 MHA sequences, 128 GQA sequences with lognormal lengths): the one-call
    step against the oracle's write and float64 attention."""
    wl = W.generate(cfg)
    t = upload(wl, dev)
    out = ops.decode_step(t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"], t["block_tables"],
                          t["seq_lens"], wl.scale, wl.max_seq_len)
    torch.cuda.synchronize()
    _, r_kc, r_vc, r_out = oracle_step(wl)
    assert same_bits(t["key_cache"], r_kc) and same_bits(t["value_cache"], r_vc), "cache contents differ"
    assert_attn_close(out, r_out, wl.spec.dtype, "decode_step config %d" % cfg)


@pytest.mark.parametrize("name", ["f32-gqa4-bs32", "gqa16-d64", "gqa32-d128-bs32"])
def test_step_matches_oracle_small(name, dev):
    wl = W.generate(SHAPES[name], seed=307)
    t = upload(wl, dev)
    out = ops.decode_step(t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"], t["block_tables"],
                          t["seq_lens"], wl.scale, wl.max_seq_len)
    torch.cuda.synchronize()
    _, r_kc, r_vc, r_out = oracle_step(wl)
    assert same_bits(t["key_cache"], r_kc) and same_bits(t["value_cache"], r_vc)
    assert_attn_close(out, r_out, wl.spec.dtype, name)


@pytest.mark.parametrize("name", ["gqa8-bs16", "gqa2-d64-bs32"])
def test_step_fp8_matches_oracle(name, dev):
    wl = W.generate(SHAPES[name], seed=308)
    t = upload_fp8(wl, dev)
    out = ops.decode_step_fp8(t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"],
                              t["block_tables"], t["seq_lens"], wl.scale, wl.max_seq_len, K_SCALE, V_SCALE)
    torch.cuda.synchronize()
    _, r_kc, r_vc, r_out = oracle_fp8_step(wl, t)
    assert np.array_equal(t["key_cache"].cpu().numpy(), r_kc), "K codes differ"
    assert np.array_equal(t["value_cache"].cpu().numpy(), r_vc), "V codes differ"
    assert_attn_close(out, r_out, "bf16", "fp8 " + name)
