"""GPU parity of the shared-prefix decode calls (pkv_decode_step_shared,
pkv_paged_attention_decode_shared[_fp8]: each group's shared blocks are read
once for all its members' query heads) against the float64 oracle, through
the C ABI.  The oracle knows nothing of groups: it attends every sequence
over its own block table.  Needs an MI355X and libpagedkv.so."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_97_amd import ops
from paged_kv_cache_97_amd import workloads as W
from gpu_harness import (K_SCALE, V_SCALE, assert_attn_close, log, oracle_fp8_step, oracle_step, run_step,
                         same_bits, upload, upload_fp8)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.lib()
    return torch.device("cuda:0")


def _groups(rows, dev):
    return torch.tensor(rows, dtype=torch.int32, device=dev).reshape(-1, 3)


def _written(wl, dev):
    """The workload on the GPU after the step's cache write, and the oracle's
    decode over the written pools."""
    t = upload(wl, dev)
    slots, _ = run_step(wl, t)
    _, r_kc, r_vc, r_out = oracle_step(wl)
    assert same_bits(t["key_cache"], r_kc) and same_bits(t["value_cache"], r_vc)
    return t, r_out


def test_config4_step_full_size(dev):
    """The long-context batch: 16 sequences share their first 2048 tokens (64
    blocks of 32).  One group names all of them; the fused step writes every
    new token and attends, each member's prefix read in one pass."""
    wl = W.generate(4)
    t = upload(wl, dev)
    g = _groups([0, wl.num_seqs, wl.spec.shared_prefix_tokens], dev)
    out = ops.decode_step_shared(t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"],
                                 t["block_tables"], t["seq_lens"], wl.scale, wl.max_seq_len, g)
    torch.cuda.synchronize()
    _, r_kc, r_vc, r_out = oracle_step(wl)
    assert same_bits(t["key_cache"], r_kc) and same_bits(t["value_cache"], r_vc), "cache write differs"
    assert_attn_close(out, r_out, "bf16", "config 4 shared step")


SPEC = W.reduced(4, num_decode=12, decode_len=("uniform", 300, 1500), shared_prefix_tokens=256)
SPEC16 = W.reduced(3, num_decode=10, decode_len=("uniform", 200, 900), shared_prefix_tokens=160)


@pytest.mark.parametrize("groups", [
    [0, 12, 256],                              # everyone, the whole prefix
    [0, 5, 256, 5, 7, 128],                    # two groups, the second claims a shorter prefix
    [2, 3, 256, 7, 1, 256],                    # partial membership, a group of one
    [0, 12, 200],                              # not a multiple of 16: rounded down to 192
    [0, 12, 96, 0, 12, 256],                   # overlapping groups (exact, repeated work)
])
def test_groups_against_oracle(groups, dev):
    wl = W.generate(SPEC, seed=61)
    t, r_out = _written(wl, dev)
    out = ops.paged_attention_decode_shared(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                            t["seq_lens"], wl.scale, wl.max_seq_len, _groups(groups, dev))
    torch.cuda.synchronize()
    assert_attn_close(out, r_out, "bf16", "groups %s" % groups)


@pytest.mark.parametrize("name,spec", [
    ("gqa4-bs32-d128", SPEC),
    ("gqa8-bs16-d128", SPEC16),
    ("gqa3-bs16-d128", W.reduced(3, num_decode=11, num_q_heads=12, num_kv_heads=4, decode_len=("uniform", 100, 600),
                                 shared_prefix_tokens=64)),
    ("gqa16-bs16-d64", W.reduced(3, num_decode=6, num_q_heads=32, num_kv_heads=2, head_dim=64,
                                 decode_len=("uniform", 64, 700), shared_prefix_tokens=48)),
    ("mha-bs32-d64", W.reduced(2, num_decode=9, num_q_heads=8, num_kv_heads=8, head_dim=64, block_size=32,
                               pool_blocks=None, decode_len=("uniform", 70, 400), shared_prefix_tokens=64)),
])
@pytest.mark.parametrize("workers,dyn", [(0, -1), (3, 0), (333, 120), (0, 500)])
def test_shapes_and_splits(name, spec, workers, dyn, dev):
    """Group sizes whose columns straddle column blocks (G = 3), many column
    blocks (G = 16), MHA, head_dim 64/128, blocks of 16/32, few and many
    workers, static and unit splits: the fused step equals the oracle."""
    prev_w, prev_d = ops.set_decode_workers(workers), ops.set_decode_dynamic(dyn, 2)
    try:
        wl = W.generate(spec, seed=62)
        log("[shared %s] workers %d dyn %d: B=%d maxL=%d" % (name, workers, dyn, wl.num_seqs, wl.max_seq_len))
        t = upload(wl, dev)
        out = ops.decode_step_shared(t["query"], t["key"], t["value"], t["key_cache"], t["value_cache"],
                                     t["block_tables"], t["seq_lens"], wl.scale, wl.max_seq_len,
                                     _groups([0, wl.num_seqs, spec.shared_prefix_tokens], dev))
        torch.cuda.synchronize()
        _, r_kc, r_vc, r_out = oracle_step(wl)
        assert same_bits(t["key_cache"], r_kc) and same_bits(t["value_cache"], r_vc)
        assert_attn_close(out, r_out, "bf16", name)
    finally:
        ops.set_decode_workers(prev_w)
        ops.set_decode_dynamic(prev_d, 4)


def test_members_shorter_than_the_prefix(dev):
    """Attention-only call with members whose seq_lens end inside the shared
    prefix (they attend only their own tokens, with per-column masks in the
    prefix pass), one of them empty."""
    wl = W.generate(SPEC, seed=63)
    t, _ = _written(wl, dev)
    sl = wl.seq_lens.copy()
    sl[[1, 4, 9]] = [17, 1, 250]
    sl[6] = 0
    _, r_kc, r_vc, _ = oracle_step(wl)
    r_out = oracle.decode_attention(wl.query, r_kc, r_vc, wl.block_tables, sl, wl.scale, "bf16")
    out = ops.paged_attention_decode_shared(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                            torch.from_numpy(sl).to(dev), wl.scale, int(sl.max()),
                                            _groups([0, 12, 256], dev))
    torch.cuda.synchronize()
    assert not out[6].any(), "an empty sequence gives a zero row"
    assert_attn_close(out, r_out, "bf16", "short members")


def test_fp8_pools(dev):
    wl = W.generate(SPEC, seed=64)
    t = upload_fp8(wl, dev)
    slots = torch.empty(wl.num_tokens, dtype=torch.int64, device=dev)
    ops.write_new_tokens_fp8(t["block_tables"], t["positions"], t["query_start_loc"], wl.spec.block_size, t["key"],
                             t["value"], t["key_cache"], t["value_cache"], K_SCALE, V_SCALE, slots)
    out = ops.paged_attention_decode_shared_fp8(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                                t["seq_lens"], wl.scale, wl.max_seq_len, K_SCALE, V_SCALE,
                                                _groups([0, 12, 256], dev))
    torch.cuda.synchronize()
    _, r_kc, r_vc, r_out = oracle_fp8_step(wl, t)
    assert np.array_equal(t["key_cache"].cpu().numpy(), r_kc)
    assert_attn_close(out, r_out, "bf16", "fp8 shared")


def test_deterministic_and_equal_to_the_plain_call_within_tolerance(dev):
    """Two shared calls give the same bits (fixed parts and merge order); the
    plain call over the same pools agrees within the bf16 tolerance."""
    wl = W.generate(4)
    t, r_out = _written(wl, dev)
    g = _groups([0, wl.num_seqs, 2048], dev)
    a = ops.paged_attention_decode_shared(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                          t["seq_lens"], wl.scale, wl.max_seq_len, g)
    b = ops.paged_attention_decode_shared(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                          t["seq_lens"], wl.scale, wl.max_seq_len, g)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert_attn_close(a, r_out, "bf16", "config 4 shared attention")


def test_rejected_on_the_host(dev):
    wl = W.generate(SPEC, seed=65)
    t = upload(wl, dev)
    with pytest.raises(ops.PagedKVError, match="EUNSUPPORTED"):
        ops.paged_attention_decode_shared(t["query"].float(), t["key_cache"].float(), t["value_cache"].float(),
                                          t["block_tables"], t["seq_lens"], wl.scale, wl.max_seq_len,
                                          _groups([0, 12, 256], dev))
