"""CPU oracle for the paged KV-cache hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy.  It shares no code with the HIP library or its
Python binding and imports nothing from them.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does.

What it computes, and where the pages state it:
  * slot_mapping -- gaoleia.github.io "PagedAttention 和 Continuous Batching"
    §1.5 Slot Mapping: logical block = position // block_size, offset =
    position % block_size, slot = block_table[logical block] * block_size +
    offset (worked example: position 35, block_size 16, table entry 9 -> 147).
  * reshape_and_cache -- feifeigd.github.io "vLLM 架构详解" 一 PagedAttention
    (append_token writes a token's K/V at its in-block position of the last
    block) and gaoleia §1.3 (a block holds K and V as [block_size, heads,
    head_dim]) and §2.4 (a decode step appends K6,V6 before attending).
  * attention -- gaoleia §1.6: gather K and V of the sequence's blocks in
    logical order, keep the first seq_len tokens, then softmax(q K^T / sqrt(d))
    V.  Paging only moves where K/V live, so this is exact dense attention.
  * copy_blocks / swap_blocks -- lakecityint.com/news/209622 §3.2 (copy-on-
    write: a new physical block receives a copy of the shared block before
    one sharer writes) and §2.1, 5688vip.com "vLLM核心机制" §3.3 (preemption
    swaps a sequence's blocks out to CPU memory and back in later).
  * FP8 KV cache -- feifeigd "vLLM 架构详解" 三 生产级部署配置, 关键参数调优
    (kv-cache-dtype auto or fp8: fp8 halves KV memory at a small loss of
    precision).  The pages name no format or scale; the reading taken here is
    OCP FP8 E4M3 (bias 7, no infinities, S.1111.111 is NaN, largest finite
    448, subnormals m/8 * 2^-6) with one float scale per pool: a value x is
    stored as the E4M3 code nearest to float32(x) * float32(1 / scale) (ties
    to the even code, magnitudes past 448 saturate to 448) and read back as
    E4M3 value * scale.
  * varlen rows -- gaoleia §2.4 (one iteration mixes decode rows and prefill
    rows) and §2.5 (a long prompt is cut into 512-token chunks interleaved
    with decodes); fanquanpp.github.io "vLLM服务内部" 分块预填充.  A chunk of q
    rows with c earlier tokens: row i sits at position c + i and sees keys
    0..c+i (causal mask aligned to the end of the key range).

Readings taken where the pages are silent (each is also tested):
  * GQA: query head h reads KV head h // (Hq / Hkv).
  * seq_len 0 gives a zero output row; a sequence with no query rows has none.
  * positions < 0 map to slot -1, and slot -1 is not written.
  * slots >= seq_len inside the last block never contribute, whatever they hold.

Parity pins live in tests/test_oracle_pins.py; every function here has at
least one pin that does not restate its formula.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to_f64", "slot_mapping", "reshape_and_cache", "gather_tokens",
    "decode_attention", "varlen_attention", "attention_rows",
    "partial_attention", "combine_partials", "copy_blocks", "swap_blocks",
    "e4m3_value", "e4m3_encode", "quantize_kv", "reshape_and_cache_fp8",
]


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values: bf16 bit patterns (uint16) are the top
    half of a float32; fp32 values widen as they are."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError("dtype must be 'bf16' or 'f32'")


def slot_mapping(block_tables, positions, query_start_loc, block_size, num_blocks=None):
    """Physical slot of every new token (gaoleia §1.5).

    Token t belongs to the sequence s with qsl[s] <= t < qsl[s+1]; its slot is
    block_tables[s][pos // bs] * bs + pos % bs, or -1 when pos < 0.
    """
    bt = np.asarray(block_tables)
    pos = np.asarray(positions)
    qsl = np.asarray(query_start_loc)
    out = np.full(pos.shape[0], -1, dtype=np.int64)
    for s in range(qsl.shape[0] - 1):
        for t in range(int(qsl[s]), int(qsl[s + 1])):
            p = int(pos[t])
            if p < 0:
                continue
            logical_block = p // block_size
            offset = p % block_size
            assert logical_block < bt.shape[1], "position beyond the block table"
            physical_block = int(bt[s, logical_block])
            assert physical_block >= 0, "position in an unallocated logical block"
            if num_blocks is not None:
                assert physical_block < num_blocks, "block id outside the pool"
            out[t] = physical_block * block_size + offset
    return out


def reshape_and_cache(key, value, key_cache, value_cache, slots, ref_counts=None):
    """Copy each new token's K and V rows, bit for bit, into its slot.

    Returns new cache arrays; every other byte is unchanged.  Slots must be
    unique (two writers of one slot would race), and a block shared by several
    tables (ref_count > 1) must not be written (it needs copy-on-write first).
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    bs = kc.shape[1]
    live = [int(s) for s in np.asarray(slots) if s >= 0]
    assert len(live) == len(set(live)), "duplicate slots"
    for t, slot in enumerate(np.asarray(slots)):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = slot // bs, slot % bs
        if ref_counts is not None:
            assert ref_counts[block] <= 1, "write into a shared block"
        kc[block, offset] = key[t]
        vc[block, offset] = value[t]
    return kc, vc


def gather_tokens(cache, table_row, length, block_size):
    """Rows [length, Hkv, D] of one sequence in logical order, each found
    through the block table (gaoleia §1.6 step 1 and step 4)."""
    rows = np.empty((length,) + cache.shape[2:], dtype=cache.dtype)
    for p in range(length):
        block = int(table_row[p // block_size])
        assert block >= 0
        rows[p] = cache[block, p % block_size]
    return rows


def attention_rows(q, k, v, scale, visible):
    """Softmax attention of query rows over key rows, float64.

    q [R, D], k [L, D], v [L, D]; row r attends keys 0..visible[r]-1.
    A row with no visible key gives zeros.
    """
    R, L = q.shape[0], k.shape[0]
    visible = np.asarray(visible, dtype=np.int64).reshape(R)
    assert np.all((visible >= 0) & (visible <= L))
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    rows = visible > 0
    if not rows.any() or L == 0:
        return out
    scores = scale * (q[rows] @ k.T)                  # [R', L]
    mask = np.arange(L)[None, :] < visible[rows][:, None]
    x = np.where(mask, scores, -np.inf)
    m = x.max(axis=1, keepdims=True)
    w = np.where(mask, np.exp(x - m), 0.0)
    out[rows] = (w / w.sum(axis=1, keepdims=True)) @ v
    return out


def _kv_rows(cache, table_row, length, block_size, dtype, kv_scale):
    rows = gather_tokens(cache, table_row, length, block_size)
    if kv_scale is None:
        return to_f64(rows, dtype)
    return e4m3_value(rows) * float(kv_scale)


def decode_attention(query, key_cache, value_cache, block_tables, seq_lens, scale, dtype, kv_scales=None):
    """One query row per sequence over its first seq_lens[s] cached tokens.

    query [B, Hq, D]; caches [NB, bs, Hkv, D]; returns float64 [B, Hq, D].
    kv_scales = (k_scale, v_scale) means the caches hold E4M3 codes, read as
    code value * scale; the query stays in `dtype`.
    """
    B, Hq, D = query.shape
    Hkv = key_cache.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    bs = key_cache.shape[1]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in range(B):
        L = int(seq_lens[s])
        if L == 0:
            continue
        ks, vs = kv_scales if kv_scales is not None else (None, None)
        k = _kv_rows(key_cache, block_tables[s], L, bs, dtype, ks)
        v = _kv_rows(value_cache, block_tables[s], L, bs, dtype, vs)
        q = to_f64(query[s], dtype)
        for h in range(Hq):
            g = h // group
            out[s, h] = attention_rows(q[h:h + 1], k[:, g], v[:, g], scale, [L])[0]
    return out


def varlen_attention(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, scale, dtype,
                     kv_scales=None):
    """Mixed prefill-chunk and decode rows in one step.

    Sequence s owns rows qsl[s]..qsl[s+1]-1 (q_s of them); row i sits at
    position seq_lens[s] - q_s + i and attends keys 0..that position.
    query [T, Hq, D]; returns float64 [T, Hq, D].  kv_scales as in
    decode_attention.
    """
    T, Hq, D = query.shape
    Hkv = key_cache.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    bs = key_cache.shape[1]
    out = np.zeros((T, Hq, D), dtype=np.float64)
    qsl = np.asarray(query_start_loc)
    for s in range(qsl.shape[0] - 1):
        r0, r1 = int(qsl[s]), int(qsl[s + 1])
        nq = r1 - r0
        if nq == 0:
            continue
        L = int(seq_lens[s])
        assert L >= nq, "fewer keys than query rows"
        visible = [L - nq + i + 1 for i in range(nq)]
        ks, vs = kv_scales if kv_scales is not None else (None, None)
        k = _kv_rows(key_cache, block_tables[s], L, bs, dtype, ks)
        v = _kv_rows(value_cache, block_tables[s], L, bs, dtype, vs)
        q = to_f64(query[r0:r1], dtype)
        for h in range(Hq):
            g = h // group
            out[r0:r1, h] = attention_rows(q[:, h], k[:, g], v[:, g], scale, visible)
    return out


def partial_attention(q, k, v, scale):
    """Unnormalised state of one part of the key range: the part's max score
    m, its sum Z of exp(x - m), and sum_j exp(x_j - m) v_j."""
    x = scale * (k @ q)
    m = x.max()
    w = np.exp(x - m)
    return m, w.sum(), w @ v


def combine_partials(parts):
    """Merge part states (m_k, Z_k, o_k) of disjoint key ranges into the
    attention output: weights exp(m_k - M) with M the largest m_k."""
    M = max(p[0] for p in parts)
    Z = sum(np.exp(m - M) * z for m, z, _ in parts)
    o = sum(np.exp(m - M) * ok for m, _, ok in parts)
    return o / Z


def _check_mapping(mapping, n_src, n_dst, same_pool):
    pairs = [(int(a), int(b)) for a, b in np.asarray(mapping).reshape(-1, 2)]
    dsts = [b for _, b in pairs]
    assert len(dsts) == len(set(dsts)), "two copies into one block"
    assert all(0 <= a < n_src and 0 <= b < n_dst for a, b in pairs), "block id outside the pool"
    if same_pool:
        assert not set(dsts) & {a for a, _ in pairs}, "a destination is also a source"
    return pairs


def copy_blocks(key_cache, value_cache, mapping):
    """Copy-on-write block copies inside the pools (lakecityint §3.2): for
    each (src, dst) pair block dst becomes a bit copy of block src, K and V.
    Destinations are distinct and are not sources of the same call."""
    pairs = _check_mapping(mapping, key_cache.shape[0], key_cache.shape[0], True)
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    for src, dst in pairs:
        kc[dst] = key_cache[src]
        vc[dst] = value_cache[src]
    return kc, vc


def swap_blocks(src_pool, dst_pool, mapping):
    """Swap-out / swap-in of whole blocks between two pools (GPU <-> CPU;
    5688vip §3.3, lakecityint §2.1): block dst of dst_pool becomes a bit copy
    of block src of src_pool."""
    pairs = _check_mapping(mapping, src_pool.shape[0], dst_pool.shape[0], False)
    out = np.array(dst_pool, copy=True)
    for src, dst in pairs:
        out[dst] = src_pool[src]
    return out


# ---------------------------------------------------------------- FP8 (OCP E4M3)
def e4m3_value(codes) -> np.ndarray:
    """Value of each E4M3 byte as float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_value(np.arange(0x7F))          # codes 0x00..0x7E, increasing magnitudes


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each float (ties to the even code; magnitudes of
    448 and more give 448).  Inputs must not be NaN."""
    v = np.asarray(v, dtype=np.float64)
    assert not np.isnan(v).any(), "NaN has no saturating code"
    a = np.minimum(np.abs(v), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _E4M3_POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_kv(x, dtype, kv_scale) -> np.ndarray:
    """E4M3 codes of stored values x (bf16 bits or float32): the float32
    product of x and the float32 reciprocal of the scale, rounded once."""
    inv = np.float32(1.0) / np.float32(kv_scale)
    xf = to_f64(x, dtype).astype(np.float32)
    return e4m3_encode((xf * inv).astype(np.float32))


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slots, k_scale, v_scale, dtype, ref_counts=None):
    """reshape_and_cache into E4M3 pools: each new token's K and V rows are
    quantised (quantize_kv) and stored at its slot; nothing else changes."""
    kq = quantize_kv(key, dtype, k_scale)
    vq = quantize_kv(value, dtype, v_scale)
    return reshape_and_cache(kq, vq, key_cache, value_cache, slots, ref_counts)
