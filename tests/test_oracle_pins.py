"""Pins for the float64 oracle: each check comes from something other than the
oracle's own formula -- the pages' printed examples, textbook attention from a
different library, closed forms, invariances and brute force.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_97_amd import workloads as W
from paged_kv_cache_97_amd.blocks import BlockPool, SeqBlocks


def _after_write(wl):
    slots = oracle.slot_mapping(wl.block_tables, wl.positions, wl.query_start_loc,
                                wl.spec.block_size, wl.num_blocks)
    kc, vc = oracle.reshape_and_cache(wl.key, wl.value, wl.key_cache, wl.value_cache, slots, wl.ref_counts)
    return slots, kc, vc


def _small(cfg, **kw):
    return W.reduced(cfg, **kw)


SMALL_DECODE = _small(3, num_decode=5, num_q_heads=8, num_kv_heads=2, head_dim=32,
                      decode_len=("lognormal", 60.0, W.LOGNORMAL_SIGMA, 1, 200))
SMALL_VARLEN = _small(5, num_decode=3, num_prefill=2, prefill_chunk=24, num_q_heads=4, num_kv_heads=2,
                      head_dim=16, prefill_ctx=("uniform", 0, 70),
                      decode_len=("lognormal", 40.0, W.LOGNORMAL_SIGMA, 16, 120))


# ---------------------------------------------------------------- P1 printed example
def test_slot_mapping_worked_example(golden):
    ex = golden["slot_mapping"][0]
    bt = np.array([ex["block_table"]], dtype=np.int32)
    got = oracle.slot_mapping(bt, np.array([ex["position"]]), np.array([0, 1]), ex["block_size"])
    assert got.tolist() == [ex["slot"]]
    # the intermediate quantities the page prints
    assert ex["position"] // ex["block_size"] == ex["logical_block"]
    assert ex["position"] % ex["block_size"] == ex["offset_in_block"]
    assert ex["block_table"][ex["logical_block"]] == ex["physical_block"]


def test_slot_mapping_negative_position_is_padding():
    bt = np.array([[3, 1]], dtype=np.int32)
    got = oracle.slot_mapping(bt, np.array([-1, 0, 17]), np.array([0, 3]), 16)
    assert got.tolist() == [-1, 48, 17]


# ---------------------------------------------------------------- P2 brute force
@pytest.mark.parametrize("bs", [16, 32])
def test_slot_mapping_matches_token_by_token_append(bs, golden):
    """Simulate appending tokens one at a time (the append_token process of
    the feifeigd page): a counter tracks the fill of the last block and a new
    block is taken when it is full.  Record where every token landed and
    compare with the oracle's slot for that (sequence, position)."""
    rng = np.random.default_rng(7)
    pool = BlockPool(64, order=rng.permutation(64))
    lens = [1, bs - 1, bs, bs + 1, 3 * bs + 5]
    landed = []
    tables = []
    for L in lens:
        t = SeqBlocks(bs)
        fill = bs       # "last block full" so the first token allocates
        where = []
        for _ in range(L):
            if fill == bs:
                t.append_block(pool.alloc())
                fill = 0
            where.append((t.mapping[-1], fill))
            fill += 1
        t.num_tokens = L
        tables.append(t)
        landed.append(where)
    width = max(len(t.mapping) for t in tables)
    bt = np.array([t.row(width) for t in tables], dtype=np.int32)
    positions = np.concatenate([np.arange(L) for L in lens])
    qsl = np.concatenate([[0], np.cumsum(lens)])
    slots = oracle.slot_mapping(bt, positions, qsl, bs, 64)
    expect = [blk * bs + off for where in landed for (blk, off) in where]
    assert slots.tolist() == expect
    assert len(set(expect)) == len(expect)          # injective over private tables
    for ex in golden["block_tables_printed"]:
        tbl = np.array([ex["block_table"]], dtype=np.int32)
        n = len(ex["block_table"]) * 16
        s = oracle.slot_mapping(tbl, np.arange(n), np.array([0, n]), 16)
        # consecutive positions fill each listed block in order, 16 at a time
        assert s.reshape(-1, 16).tolist() == [[b * 16 + i for i in range(16)] for b in ex["block_table"]]


def test_reshape_and_cache_copies_bits_and_nothing_else():
    wl = W.generate(1)
    slots, kc, vc = _after_write(wl)
    bs = wl.spec.block_size
    changed_k = np.zeros(kc.shape[:2], dtype=bool)
    for t, slot in enumerate(slots):
        b, o = divmod(int(slot), bs)
        assert kc[b, o].tobytes() == wl.key[t].tobytes()
        assert vc[b, o].tobytes() == wl.value[t].tobytes()
        changed_k[b, o] = True
    assert kc[~changed_k].tobytes() == wl.key_cache[~changed_k].tobytes()
    assert vc[~changed_k].tobytes() == wl.value_cache[~changed_k].tobytes()


def test_reshape_and_cache_skips_padding_and_rejects_duplicates():
    kc = np.zeros((2, 4, 1, 2), np.float32)
    key = np.ones((2, 1, 2), np.float32)
    out_k, _ = oracle.reshape_and_cache(key, key, kc, kc, np.array([-1, 5]))
    assert out_k.reshape(8, 2)[5].tolist() == [1, 1] and out_k.sum() == 2
    with pytest.raises(AssertionError):
        oracle.reshape_and_cache(key, key, kc, kc, np.array([5, 5]))


def test_write_into_shared_block_is_refused():
    kc = np.zeros((2, 4, 1, 2), np.float32)
    key = np.ones((1, 1, 2), np.float32)
    with pytest.raises(AssertionError):
        oracle.reshape_and_cache(key, key, kc, kc, np.array([1]), ref_counts=[2, 1])


# ---------------------------------------------------------------- P5 dense equality
def _sdpa_reference(q_rows, k_all, v_all, scale, visible, group):
    """torch float64 scaled_dot_product_attention over contiguous K/V with an
    explicit mask and KV heads repeated for GQA.  q_rows [R, Hq, D],
    k_all/v_all [L, Hkv, D] (float64)."""
    q = torch.from_numpy(q_rows).permute(1, 0, 2)                      # [Hq, R, D]
    k = torch.from_numpy(k_all).permute(1, 0, 2).repeat_interleave(group, 0)
    v = torch.from_numpy(v_all).permute(1, 0, 2).repeat_interleave(group, 0)
    L = k.shape[1]
    mask = torch.arange(L)[None, :] < torch.tensor(visible)[:, None]   # [R, L]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("seed", [11, 12])
def test_decode_equals_dense_attention(seed):
    wl = W.generate(SMALL_DECODE, seed=seed, keep_logical=True)
    _, kc, vc = _after_write(wl)
    got = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, "bf16")
    G = wl.spec.num_q_heads // wl.spec.num_kv_heads
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        ref = _sdpa_reference(oracle.to_f64(wl.query[s:s + 1], "bf16"),
                              oracle.to_f64(wl.logical_k[s], "bf16"),
                              oracle.to_f64(wl.logical_v[s], "bf16"), wl.scale, [L], G)
        np.testing.assert_allclose(got[s], ref[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [21, 22])
def test_varlen_equals_dense_attention_bottom_right_causal(seed):
    wl = W.generate(SMALL_VARLEN, seed=seed, keep_logical=True)
    _, kc, vc = _after_write(wl)
    got = oracle.varlen_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                  wl.scale, "bf16")
    G = wl.spec.num_q_heads // wl.spec.num_kv_heads
    qsl = wl.query_start_loc
    for s in range(wl.num_seqs):
        r0, r1 = int(qsl[s]), int(qsl[s + 1])
        L = int(wl.seq_lens[s])
        ctx = L - (r1 - r0)
        visible = [ctx + i + 1 for i in range(r1 - r0)]
        ref = _sdpa_reference(oracle.to_f64(wl.query[r0:r1], "bf16"),
                              oracle.to_f64(wl.logical_k[s], "bf16"),
                              oracle.to_f64(wl.logical_v[s], "bf16"), wl.scale, visible, G)
        np.testing.assert_allclose(got[r0:r1], ref, rtol=0, atol=1e-12)


def test_fp32_tiny_config_equals_dense_attention():
    wl = W.generate(1, keep_logical=True)
    _, kc, vc = _after_write(wl)
    got = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, "f32")
    for s in range(2):
        ref = _sdpa_reference(wl.query[s:s + 1].astype(np.float64), wl.logical_k[s].astype(np.float64),
                              wl.logical_v[s].astype(np.float64), 1.0 / 8.0, [int(wl.seq_lens[s])], 1)
        np.testing.assert_allclose(got[s], ref[0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P6 closed forms
def _one_seq_pool(k_rows, v_rows, bs=16, seed=0, poison=np.nan):
    """Place one sequence's rows [L, Hkv, D] (float32) into a shuffled pool."""
    L = k_rows.shape[0]
    nb = -(-L // bs)
    NB = nb + 3
    order = np.random.default_rng(seed).permutation(NB)
    table = order[:nb]
    kc = np.full((NB, bs) + k_rows.shape[1:], poison, np.float32)
    vc = np.full_like(kc, poison)
    for lb, b in enumerate(table):
        n = min(bs, L - lb * bs)
        kc[b, :n] = k_rows[lb * bs: lb * bs + n]
        vc[b, :n] = v_rows[lb * bs: lb * bs + n]
    return kc, vc, np.array([table], dtype=np.int32)


def test_zero_keys_give_mean_of_values_and_catch_missing_tokens():
    L, D = 37, 8
    v = np.zeros((L, 1, D), np.float32)
    v[:, 0, 0] = np.arange(L)             # exact integers
    v[:, 0, 1] = np.arange(L) % 5
    kc, vc, bt = _one_seq_pool(np.zeros_like(v), v)
    q = np.random.default_rng(1).standard_normal((1, 1, D)).astype(np.float32)
    o = oracle.decode_attention(q, kc, vc, bt, np.array([L]), 0.3, "f32")
    assert o[0, 0, 0] == pytest.approx((L - 1) / 2, abs=1e-12)
    assert o[0, 0, 1] == pytest.approx(np.mean(np.arange(L) % 5), abs=1e-12)


def test_single_token_returns_its_value_and_constant_values_are_fixed_points():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((1, 2, 4)).astype(np.float32)
    v = rng.standard_normal((1, 2, 4)).astype(np.float32)
    kc, vc, bt = _one_seq_pool(k, v)
    q = rng.standard_normal((1, 4, 4)).astype(np.float32)
    o = oracle.decode_attention(q, kc, vc, bt, np.array([1]), 0.5, "f32")
    assert np.array_equal(o[0, :2], np.repeat(v[0, :1].astype(np.float64), 2, 0))
    assert np.array_equal(o[0, 2:], np.repeat(v[0, 1:].astype(np.float64), 2, 0))
    L = 50
    k = rng.standard_normal((L, 1, 4)).astype(np.float32)
    v = np.full((L, 1, 4), 1.25, np.float32)
    kc, vc, bt = _one_seq_pool(k, v)
    o = oracle.decode_attention(q[:, :1], kc, vc, bt, np.array([L]), 0.5, "f32")
    np.testing.assert_allclose(o, 1.25, rtol=0, atol=1e-14)


def test_two_keys_logistic_weight_pins_scale_and_sign():
    """Scores x0 = scale*a, x1 = 0 give weight 1/(1+exp(-scale*a)) on V0."""
    a, scale = 3.0, 0.7
    k = np.zeros((2, 1, 2), np.float32)
    k[0, 0, 0] = a
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], np.float32)
    kc, vc, bt = _one_seq_pool(k, v)
    q = np.array([[[1.0, 0.0]]], np.float32)
    o = oracle.decode_attention(q, kc, vc, bt, np.array([2]), scale, "f32")
    w0 = 1.0 / (1.0 + math.exp(-scale * a))
    np.testing.assert_allclose(o[0, 0], [w0, 1 - w0], rtol=0, atol=1e-15)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(3)
    L, D = 40, 16
    k = rng.standard_normal((L, 1, D)).astype(np.float32)
    q = rng.standard_normal(D).astype(np.float32)
    k[17, 0] = 40.0 * q / np.linalg.norm(q) * np.sqrt(D)
    v = rng.standard_normal((L, 1, D)).astype(np.float32)
    kc, vc, bt = _one_seq_pool(k, v)
    o = oracle.decode_attention(q.reshape(1, 1, D), kc, vc, bt, np.array([L]), 1 / np.sqrt(D), "f32")
    np.testing.assert_allclose(o[0, 0], v[17, 0], rtol=0, atol=1e-6)


def test_poisoned_slots_beyond_seq_len_never_contribute():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((21, 2, 8)).astype(np.float32)
    v = rng.standard_normal((21, 2, 8)).astype(np.float32)
    q = rng.standard_normal((1, 2, 8)).astype(np.float32)
    a = oracle.decode_attention(q, *_one_seq_pool(k, v, poison=np.nan), np.array([21]), 0.3, "f32")
    kc, vc, bt = _one_seq_pool(k, v, poison=0.0)
    b = oracle.decode_attention(q, kc, vc, bt, np.array([21]), 0.3, "f32")
    assert np.isfinite(a).all() and np.array_equal(a, b)


def test_empty_sequence_gives_zero_row_and_no_query_rows_gives_nothing():
    kc = np.full((2, 16, 1, 4), np.nan, np.float32)
    q = np.ones((2, 1, 4), np.float32)
    bt = np.array([[0], [-1]], dtype=np.int32)
    kc[0, :3] = 1.0
    o = oracle.decode_attention(q, kc, kc, bt, np.array([3, 0]), 1.0, "f32")
    assert np.array_equal(o[1], np.zeros((1, 4))) and np.allclose(o[0], 1.0)
    ov = oracle.varlen_attention(q[:1], kc, kc, bt, np.array([3, 0]), np.array([0, 1, 1]), 1.0, "f32")
    assert ov.shape == (1, 1, 4) and np.allclose(ov, 1.0)


# ---------------------------------------------------------------- P3/P4 invariances
def test_block_permutation_invariance_is_bitwise():
    wl = W.generate(SMALL_DECODE, seed=31)
    _, kc, vc = _after_write(wl)
    ref = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, "bf16")
    perm = np.random.default_rng(5).permutation(wl.num_blocks)     # new id of block b is perm[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    got = oracle.decode_attention(wl.query, kc2, vc2, bt2, wl.seq_lens, wl.scale, "bf16")
    assert np.array_equal(ref, got)


def test_shared_prefix_equals_private_copies_bitwise():
    spec = _small(4, num_decode=4, num_q_heads=4, num_kv_heads=2, head_dim=16,
                  decode_len=("uniform", 70, 130), shared_prefix_tokens=64)
    wl = W.generate(spec, seed=41)
    _, kc, vc = _after_write(wl)
    bs = spec.block_size
    shared = [int(b) for b in wl.block_tables[0, :64 // bs]]
    assert all(wl.ref_counts[b] == wl.num_seqs for b in shared)
    ref = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, "bf16")
    # give every sequence after the first its own copy of the prefix blocks
    extra = (wl.num_seqs - 1) * len(shared)
    kc2 = np.concatenate([kc, np.zeros((extra,) + kc.shape[1:], kc.dtype)])
    vc2 = np.concatenate([vc, np.zeros((extra,) + vc.shape[1:], vc.dtype)])
    bt2 = wl.block_tables.copy()
    nxt = kc.shape[0]
    for s in range(1, wl.num_seqs):
        for i, b in enumerate(shared):
            kc2[nxt] = kc[b]
            vc2[nxt] = vc[b]
            bt2[s, i] = nxt
            nxt += 1
    got = oracle.decode_attention(wl.query, kc2, vc2, bt2, wl.seq_lens, wl.scale, "bf16")
    assert np.array_equal(ref, got)


def test_gqa_equals_expanded_mha():
    wl = W.generate(SMALL_DECODE, seed=51)
    _, kc, vc = _after_write(wl)
    G = wl.spec.num_q_heads // wl.spec.num_kv_heads
    ref = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, "bf16")
    kx = np.repeat(kc, G, axis=2)          # head g*G + j of the MHA pool is a copy of KV head g
    vx = np.repeat(vc, G, axis=2)
    got = oracle.decode_attention(wl.query, kx, vx, wl.block_tables, wl.seq_lens, wl.scale, "bf16")
    assert np.array_equal(ref, got)


# ---------------------------------------------------------------- P8/P9 varlen consistency
def test_varlen_decode_rows_equal_decode_and_follow_sequence_order():
    wl = W.generate(SMALL_VARLEN, seed=61)
    _, kc, vc = _after_write(wl)
    out = oracle.varlen_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                  wl.scale, "bf16")
    dec = np.where(~wl.is_prefill)[0]
    rows = wl.query_start_loc[dec]
    ref = oracle.decode_attention(wl.query[rows], kc, vc, wl.block_tables[dec], wl.seq_lens[dec],
                                  wl.scale, "bf16")
    assert np.array_equal(out[rows], ref)
    # reverse the sequence order: rows move with their sequence
    order = np.arange(wl.num_seqs)[::-1]
    qlen = wl.query_lens[order]
    qsl2 = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    q2 = np.concatenate([wl.query[wl.query_start_loc[s]:wl.query_start_loc[s + 1]] for s in order])
    out2 = oracle.varlen_attention(q2, kc, vc, wl.block_tables[order], wl.seq_lens[order], qsl2,
                                   wl.scale, "bf16")
    for i, s in enumerate(order):
        assert np.array_equal(out2[qsl2[i]:qsl2[i + 1]], out[wl.query_start_loc[s]:wl.query_start_loc[s + 1]])


def test_chunked_prefill_equals_one_pass():
    """A prompt of 64 tokens as 4 chunks of 16 (each chunk's K/V written
    before its attention) gives the rows of one causal pass over 64."""
    rng = np.random.default_rng(71)
    N, Hq, Hkv, D, bs = 64, 4, 2, 8, 16
    q = rng.standard_normal((N, Hq, D)).astype(np.float32)
    k = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    kc, vc, bt = _one_seq_pool(k, v, bs=bs)
    one = oracle.varlen_attention(q, kc, vc, bt, np.array([N]), np.array([0, N]), 0.35, "f32")
    empty_k = np.full_like(kc, np.nan)
    empty_v = np.full_like(vc, np.nan)
    rows = []
    for c in range(4):
        lo, hi = 16 * c, 16 * (c + 1)
        slots = oracle.slot_mapping(bt, np.arange(lo, hi), np.array([0, 16]), bs)
        empty_k, empty_v = oracle.reshape_and_cache(k[lo:hi], v[lo:hi], empty_k, empty_v, slots)
        rows.append(oracle.varlen_attention(q[lo:hi], empty_k, empty_v, bt, np.array([hi]),
                                            np.array([0, 16]), 0.35, "f32"))
    np.testing.assert_allclose(np.concatenate(rows), one, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P10 split identity
@pytest.mark.parametrize("part", [1, 7, 16, 32, 100, 1000])
def test_split_combine_identity(part):
    rng = np.random.default_rng(81)
    L, D = 300, 16
    q = rng.standard_normal(D)
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    full = oracle.attention_rows(q[None], k, v, 0.25, [L])[0]
    parts = [oracle.partial_attention(q, k[i:i + part], v[i:i + part], 0.25) for i in range(0, L, part)]
    np.testing.assert_allclose(oracle.combine_partials(parts), full, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- mistakes the pins catch
def test_pins_catch_planted_mistakes():
    """Plant plausible mistakes in copies of oracle steps (never in the HIP
    path) and check that the pins above would reject each."""
    rng = np.random.default_rng(91)
    # (1) slot = physical * bs + logical block (offset and block swapped)
    assert 9 * 16 + 35 // 16 != 147
    # (2) top-left causal alignment for a chunk after context: differs from
    #     the bottom-right rows of one pass (caught by the dense pin)
    L, nq, D = 20, 5, 4
    q, k, v = rng.standard_normal((nq, D)), rng.standard_normal((L, D)), rng.standard_normal((L, D))
    right = oracle.attention_rows(q, k, v, 0.5, [L - nq + i + 1 for i in range(nq)])
    left = oracle.attention_rows(q, k, v, 0.5, [i + 1 for i in range(nq)])
    assert not np.allclose(right, left)
    # (3) GQA map h % Hkv instead of h // G changes outputs (dense pin uses repeat_interleave)
    wl = W.generate(SMALL_DECODE, seed=92)
    _, kc, vc = _after_write(wl)
    Hkv = wl.spec.num_kv_heads
    good = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, "bf16")
    s, L, bs = 0, int(wl.seq_lens[0]), wl.spec.block_size
    kk = oracle.to_f64(oracle.gather_tokens(kc, wl.block_tables[s], L, bs), "bf16")
    vv = oracle.to_f64(oracle.gather_tokens(vc, wl.block_tables[s], L, bs), "bf16")
    qq = oracle.to_f64(wl.query[s], "bf16")
    bad = np.stack([oracle.attention_rows(qq[h:h + 1], kk[:, h % Hkv], vv[:, h % Hkv], wl.scale, [L])[0]
                    for h in range(wl.spec.num_q_heads)])
    assert not np.allclose(good[s], bad)
    # (4) swapped K and V pools
    swapped = oracle.decode_attention(wl.query, vc, kc, wl.block_tables, wl.seq_lens, wl.scale, "bf16")
    assert not np.allclose(good, swapped)
    # (5) dropping one token (seq_len - 1)
    short = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens - 1, wl.scale, "bf16")
    assert not np.allclose(good, short, atol=1e-9)


# ---------------------------------------------------------------- P9 copy-on-write and swap
import fork_scenario as FS  # noqa: E402


def _run_scenario_oracle(sc, skip_copies=False, k_only=False):
    """Apply each step of a fork scenario with the oracle; returns the pools
    and the per-step attention outputs."""
    kc, vc = sc.key_cache, sc.value_cache
    outs = []
    for st in sc.steps:
        if st.copies and not skip_copies:
            k2, v2 = oracle.copy_blocks(kc, vc, np.array(st.copies))
            kc, vc = (k2, vc) if k_only else (k2, v2)
        slots = oracle.slot_mapping(st.block_tables, st.positions, st.query_start_loc, sc.block_size, sc.num_blocks)
        kc, vc = oracle.reshape_and_cache(st.key, st.value, kc, vc, slots,
                                          None if skip_copies else st.ref_counts)
        outs.append(oracle.decode_attention(st.query, kc, vc, st.block_tables, st.seq_lens, sc.scale, sc.dtype))
    return kc, vc, outs


def _logical_attention(sc, i, s):
    """Attention of sequence s at step i over its own token list, no pool."""
    st = sc.steps[i]
    L = int(st.seq_lens[s])
    k = oracle.to_f64(sc.logical_k[s][:L], sc.dtype)
    v = oracle.to_f64(sc.logical_v[s][:L], sc.dtype)
    q = oracle.to_f64(st.query[s], sc.dtype)
    G = sc.num_q_heads // sc.num_kv_heads
    return np.stack([oracle.attention_rows(q[h:h + 1], k[:, h // G], v[:, h // G], sc.scale, [L])[0]
                     for h in range(sc.num_q_heads)])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_on_write_keeps_every_sharer_equal_to_its_own_sequence(dtype):
    """Parent + forked children share a partly filled block; after copy-on-write
    each sequence attends exactly over its own prompt + tokens (lakecityint
    §3.2), checked bit for bit against attention over the token list itself."""
    sc = FS.build(61, dtype=dtype, head_dim=16, children=3, steps=14)
    assert len(sc.steps[0].copies) == 3 and all(not st.copies for st in sc.steps[1:])
    _, _, outs = _run_scenario_oracle(sc)
    for i in (0, 1, 10, 13):                                   # 13 crosses into a new block
        for s in range(len(sc.tables)):
            assert np.array_equal(outs[i][s], _logical_attention(sc, i, s)), (i, s)


def test_copy_blocks_copies_bits_and_leaves_other_blocks():
    rng = np.random.default_rng(62)
    kc = rng.standard_normal((9, 4, 2, 3)).astype(np.float32)
    vc = rng.standard_normal((9, 4, 2, 3)).astype(np.float32)
    kc[1, 0, 0, 0] = np.nan
    k2, v2 = oracle.copy_blocks(kc, vc, np.array([[1, 5], [1, 7], [2, 0]]))
    for src, dst in [(1, 5), (1, 7), (2, 0)]:
        assert k2[dst].tobytes() == kc[src].tobytes() and v2[dst].tobytes() == vc[src].tobytes()
    for b in (1, 2, 3, 4, 6, 8):
        assert k2[b].tobytes() == kc[b].tobytes() and v2[b].tobytes() == vc[b].tobytes()
    for bad in ([[1, 5], [2, 5]], [[1, 5], [5, 6]], [[1, 9]], [[-1, 3]]):
        with pytest.raises(AssertionError):
            oracle.copy_blocks(kc, vc, np.array(bad))


def test_swap_out_and_in_round_trip_is_bitwise():
    """Swap a sequence's blocks to a CPU pool, let other data overwrite the
    freed GPU blocks, swap back into different blocks: attention is unchanged
    bit for bit (5688vip §3.3, lakecityint §2.1)."""
    from paged_kv_cache_97_amd.blocks import swap_in, swap_out
    sc = FS.build(63, dtype="bf16", head_dim=16, children=2, steps=6)
    kc, vc, outs = _run_scenario_oracle(sc)
    st = sc.steps[-1]
    ref = outs[-1]
    child = sc.tables[1]
    cpu = BlockPool(16)
    ck = np.zeros((16,) + kc.shape[1:], kc.dtype)
    cv = np.zeros_like(ck)
    out_pairs = swap_out(child, sc.pool, cpu)
    ck = oracle.swap_blocks(kc, ck, np.array(out_pairs))
    cv = oracle.swap_blocks(vc, cv, np.array(out_pairs))
    freed = [g for g, _ in out_pairs if sc.pool.ref_count(g) == 0]   # shared prompt blocks stay
    assert 0 < len(freed) < len(out_pairs)
    kc = kc.copy()
    vc = vc.copy()
    kc[freed] = 0x7FC0                                             # reused by someone else
    vc[freed] = 0x7FC0
    in_pairs = swap_in(child, cpu, sc.pool)
    assert not set(g for _, g in in_pairs) & set(freed)
    kc_in = oracle.swap_blocks(ck, kc, np.array(in_pairs))
    vc_in = oracle.swap_blocks(cv, vc, np.array(in_pairs))
    bt = st.block_tables.copy()
    bt[1, :len(child.mapping)] = child.mapping
    got = oracle.decode_attention(st.query, kc_in, vc_in, bt, st.seq_lens, sc.scale, "bf16")
    assert np.array_equal(got, ref)
    # planted mistake: CPU blocks matched to the wrong GPU blocks on the way back
    rot = [(c, g) for (c, _), (_, g) in zip(in_pairs, in_pairs[1:] + in_pairs[:1])]
    k_bad = oracle.swap_blocks(ck, kc, np.array(rot))
    v_bad = oracle.swap_blocks(cv, vc, np.array(rot))
    bad = oracle.decode_attention(st.query, k_bad, v_bad, bt, st.seq_lens, sc.scale, "bf16")
    assert not np.array_equal(bad[1], ref[1])


def test_cow_pins_catch_planted_mistakes():
    """Skipping the copy (writing into the shared block) or copying only K
    breaks the per-sequence equality pinned above."""
    sc = FS.build(64, dtype="f32", head_dim=16, children=2, steps=2)
    _, _, skip = _run_scenario_oracle(sc, skip_copies=True)
    assert not np.array_equal(skip[0][0], _logical_attention(sc, 0, 0))
    _, _, konly = _run_scenario_oracle(sc, k_only=True)
    assert not np.array_equal(konly[0][0], _logical_attention(sc, 0, 0))


# ---------------------------------------------------------------- P10 FP8 (OCP E4M3) KV cache
def _torch_e4m3_value(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_e4m3_code(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_values_match_the_format_and_torch():
    v = oracle.e4m3_value(np.arange(256))
    t = _torch_e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(v), np.isnan(t)) and np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    # fixed points of the format: 1.0, largest normal, smallest normal and subnormal, NaN, -0
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.all(np.diff(v[:0x7F]) > 0)                      # magnitudes increase with the code


def test_e4m3_encode_rounds_to_nearest_even_like_torch():
    rng = np.random.default_rng(101)
    pos = oracle.e4m3_value(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                            # exact ties (representable in float32)
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(2000) * 1e-3, mids, -mids, near,
                        -near, pos, -pos, [0.0, 447.9, 448.0, 460.0]]).astype(np.float32)
    got = oracle.e4m3_encode(x)
    assert np.array_equal(got, _torch_e4m3_code(x))
    # ties go to the even code: halfway between 1.0 (0x38) and 1.125 (0x39) -> 0x38;
    # halfway between 1.125 and 1.25 (0x3A) -> 0x3A
    assert oracle.e4m3_encode([1.0625, 1.1875])[0] == 0x38 and oracle.e4m3_encode([1.1875])[0] == 0x3A
    # saturation (torch turns these into NaN; the reading here saturates)
    assert list(oracle.e4m3_encode([464.0, 1e6, -1e6, -500.0])) == [0x7E, 0x7E, 0xFE, 0xFE]
    # every finite code survives a round trip
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_value(finite)), np.array(finite, np.uint8))


def test_quantize_kv_is_one_float32_product_then_one_rounding():
    rng = np.random.default_rng(102)
    x = rng.standard_normal(50000).astype(np.float32)
    bits = W._to_bf16_bits(x)
    for scale in (0.0125, 1.0 / 64, 0.37):
        inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
        xf = torch.from_numpy(bits.astype(np.int32) << 16).view(torch.float32)
        ref = (xf * inv).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.quantize_kv(bits, "bf16", scale), ref)
        assert np.array_equal(oracle.quantize_kv(x, "f32", scale),
                              (torch.from_numpy(x) * inv).clamp(-448, 448).to(torch.float8_e4m3fn)
                              .view(torch.uint8).numpy())


def test_fp8_attention_equals_attention_over_dequantised_pools():
    """Decode over E4M3 pools with power-of-two scales equals, bit for bit,
    decode over float32 pools holding torch's decoding of the same codes times
    the scales; swapping the two scales is caught."""
    wl = W.generate(SMALL_DECODE, seed=103)
    _, kc, vc = _after_write(wl)
    ks, vs = 1.0 / 64, 1.0 / 32
    kq = oracle.quantize_kv(np.where(kc == W.BF16_NAN, 0, kc).astype(np.uint16), "bf16", ks)
    vq = oracle.quantize_kv(np.where(vc == W.BF16_NAN, 0, vc).astype(np.uint16), "bf16", vs)
    got = oracle.decode_attention(wl.query, kq, vq, wl.block_tables, wl.seq_lens, wl.scale, "bf16", (ks, vs))
    kf = (_torch_e4m3_value(kq) * ks).astype(np.float32)
    vf = (_torch_e4m3_value(vq) * vs).astype(np.float32)
    q32 = oracle.to_f64(wl.query, "bf16").astype(np.float32)
    ref = oracle.decode_attention(q32, kf, vf, wl.block_tables, wl.seq_lens, wl.scale, "f32")
    assert np.array_equal(got, ref)
    swapped = oracle.decode_attention(wl.query, kq, vq, wl.block_tables, wl.seq_lens, wl.scale, "bf16", (vs, ks))
    assert not np.allclose(got, swapped)


def test_fp8_write_then_decode_equals_dense_attention_of_dequantised_tokens():
    wl = W.generate(SMALL_DECODE, seed=104, keep_logical=True)
    ks, vs = 0.0125, 0.02
    slots = oracle.slot_mapping(wl.block_tables, wl.positions, wl.query_start_loc, wl.spec.block_size, wl.num_blocks)
    kc0 = np.full(wl.key_cache.shape, 0xFF, np.uint8)            # E4M3 NaN in every slot ...
    vc0 = np.full(wl.value_cache.shape, 0xFF, np.uint8)
    live = wl.key_cache != W.BF16_NAN                              # ... except cached tokens
    kc0[live] = oracle.quantize_kv(wl.key_cache[live], "bf16", ks)
    vc0[live] = oracle.quantize_kv(wl.value_cache[live], "bf16", vs)
    kc, vc = oracle.reshape_and_cache_fp8(wl.key, wl.value, kc0, vc0, slots, ks, vs, "bf16", wl.ref_counts)
    changed = np.any(kc != kc0, axis=(2, 3)) | np.any(vc != vc0, axis=(2, 3))
    written = {(int(s) // wl.spec.block_size, int(s) % wl.spec.block_size) for s in slots if s >= 0}
    assert {tuple(x) for x in np.argwhere(changed)} <= written
    got = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, "bf16", (ks, vs))
    G = wl.spec.num_q_heads // wl.spec.num_kv_heads
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        k = oracle.e4m3_value(oracle.quantize_kv(wl.logical_k[s][:L], "bf16", ks)) * ks
        v = oracle.e4m3_value(oracle.quantize_kv(wl.logical_v[s][:L], "bf16", vs)) * vs
        ref = _sdpa_reference(oracle.to_f64(wl.query[s:s + 1], "bf16"), k, v, wl.scale, [L], G)[0]
        np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- bf16 widening
def _widen_bf16_by_shift_of(x, shift):
    bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(shift)
    return bits.view(np.float32).astype(np.float64)


def _torch_bf16_to_f64(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16).double().numpy()


def _bf16_decodings_agree(ref, got):
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    return bool(np.array_equal(nan_ref, nan_got)
                and np.array_equal(ref[~nan_ref].view(np.uint64), got[~nan_got].view(np.uint64)))


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
def test_bf16_widening_equals_torch_bfloat16_on_every_bit_pattern():
    """to_f64(bits, 'bf16') is how the oracle reads every bf16 query, key and
    value.  torch's own bfloat16 -> float64 conversion decodes all 65,536 bit
    patterns: the oracle must agree bit for bit on every non-NaN pattern and on
    which patterns are NaN.  A planted widening that shifts by 8 instead of 16
    fails the same comparison."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = _torch_bf16_to_f64(bits)
    assert np.isnan(ref).sum() == 2 * 127              # exponent all ones, nonzero mantissa, both signs
    assert _bf16_decodings_agree(ref, oracle.to_f64(bits, "bf16"))
    # fixed points of the format: 1.0 = 0x3F80, -2.0 = 0xC000, +inf = 0x7F80,
    # the smallest subnormal 2^-133 = 0x0001, -0.0 = 0x8000
    fixed = {0x3F80: 1.0, 0xC000: -2.0, 0x7F80: math.inf, 0x0001: 2.0 ** -133, 0x0000: 0.0}
    for b, v in fixed.items():
        assert oracle.to_f64(np.array([b], np.uint16), "bf16")[0] == v
    assert math.copysign(1.0, oracle.to_f64(np.array([0x8000], np.uint16), "bf16")[0]) == -1.0
    assert not _bf16_decodings_agree(ref, _widen_bf16_by_shift_of(bits, 8))


def test_generator_bf16_rounding_equals_torch_cast():
    """The seeded generators round float32 normals to bf16 by round-to-nearest-
    even; torch's float32 -> bfloat16 cast is that rounding.  Checked on random
    values, on every exact tie between bf16 neighbours near 1 (both ways, both
    signs) and on the floats just beside each tie."""
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(200_000).astype(np.float32),
                        (rng.standard_normal(20_000) * 1e30).astype(np.float32),
                        (rng.standard_normal(20_000) * 1e-35).astype(np.float32)])
    # ties: float32 patterns whose low 16 bits are exactly 0x8000, plus neighbours
    hi = (np.arange(0x3F00, 0x4100, dtype=np.uint32) << 16)
    tie = hi | np.uint32(0x8000)
    ties = np.concatenate([tie, tie - 1, tie + 1, tie | np.uint32(0x80000000)]).view(np.float32)
    x = np.concatenate([x, ties])
    got = W._to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # ties to even: 1 + 2^-8 (halfway between 1.0 and 1 + 2^-7) goes down to 1.0,
    # 1 + 3 * 2^-8 goes up to 1 + 2^-6
    assert W._to_bf16_bits(np.array([1 + 2.0 ** -8], np.float32))[0] == 0x3F80
    assert W._to_bf16_bits(np.array([1 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82
