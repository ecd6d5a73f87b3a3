"""Seeded synthetic workloads for the paged KV-cache hot path.

This module only builds inputs: sequence lengths, shuffled block placement,
random query/key/value data and the pools holding the already-cached tokens.
It computes nothing of the method itself (no slot arithmetic, no attention);
both the CPU oracle and the HIP path consume what it returns.

The shapes follow the pages' workloads (no public dataset is used):
  * 16-token blocks, 128 concurrent sequences, 1500-token mean output with
    std 600 (fanquanpp.github.io "vLLM服务内部", 关键数字 and 练习 4), which
    fixes the lognormal sigma = sqrt(ln(1 + (600/1500)^2)) = 0.385;
  * 512-token prefill chunks mixed with decode rows in one step
    (gaoleia.github.io "PagedAttention 和 Continuous Batching" §2.4-§2.5);
  * long contexts and a shared system-prompt prefix held once in physical
    blocks (5688vip.com "vLLM核心机制" §3.1; feifeigd.github.io
    "vLLM 架构详解" 共享前缀的 Block 复用).

Draw order for a given seed (numpy ``default_rng``): 1 lengths, 2 the pool's
free-list permutation, 3 query, 4 cached K then cached V for every physically
distinct cached token in (sequence, position) order, 5 the step's new K then
new V.  bf16 values are float32 normals rounded to nearest even; bf16 arrays
are carried as their uint16 bit patterns.  Every pool slot that holds no valid
token is filled with NaN (bf16 0x7FC0, fp32 0x7FC00000), as a reused block
would hold stale data.

Every step writes its new tokens first: a decode sequence of length L has
L-1 cached tokens and writes token L-1; a prefill chunk of q tokens after a
context of c cached tokens writes positions c..c+q-1; seq_lens is always the
number of tokens visible to the last row (c + q).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from .blocks import BlockPool, SeqBlocks, tables_to_rows

BF16_NAN = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)
LOGNORMAL_SIGMA = math.sqrt(math.log(1.0 + (600.0 / 1500.0) ** 2))


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    dtype: str                  # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    # decode sequences: one new token each
    num_decode: int = 0
    decode_len: Tuple = ("fixed", ())          # lengths L (ctx = L - 1 ...)
    decode_len_is_ctx: bool = False            # True: the drawn value is ctx, L = ctx + 1
    # prefill chunks: q new tokens after a drawn context
    num_prefill: int = 0
    prefill_chunk: object = 512                # rows per prefill chunk (int, or one per prefill)
    prefill_ctx: Tuple = ("uniform", 0, 8192)
    prefill_first: bool = True
    # pool
    pool_blocks: Optional[int] = None          # fixed size, else slack * needed
    pool_slack: float = 1.1
    shared_prefix_tokens: int = 0              # all sequences share these blocks
    default_seed: int = 0

    def with_(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    1: WorkloadSpec("tiny-decode-f32", "f32", 4, 4, 64, 16,
                    num_decode=2, decode_len=("fixed", (35, 17)), decode_len_is_ctx=True,
                    pool_blocks=16, default_seed=1),
    2: WorkloadSpec("mha-decode-b32-bf16", "bf16", 32, 32, 128, 16,
                    num_decode=32, decode_len=("uniform", 128, 2048),
                    pool_blocks=8192, default_seed=2),
    3: WorkloadSpec("gqa-decode-b128-h64x8-bf16", "bf16", 64, 8, 128, 16,
                    num_decode=128, decode_len=("lognormal", 1500.0, LOGNORMAL_SIGMA, 16, 8192),
                    default_seed=3),
    4: WorkloadSpec("longctx-gqa-decode-b16-prefix2048-bf16", "bf16", 32, 8, 128, 32,
                    num_decode=16, decode_len=("uniform", 16384, 32768),
                    shared_prefix_tokens=2048, default_seed=4),
    5: WorkloadSpec("mixed-chunked-prefill-8x512-plus-120-decode-bf16", "bf16", 64, 8, 128, 16,
                    num_decode=120, decode_len=("lognormal", 1500.0, LOGNORMAL_SIGMA, 16, 8192),
                    decode_len_is_ctx=True,
                    num_prefill=8, prefill_chunk=512, prefill_ctx=("uniform", 0, 8192),
                    default_seed=5),
}


@dataclass
class Workload:
    spec: WorkloadSpec
    seed: int
    scale: float
    num_blocks: int
    block_tables: np.ndarray        # int32 [B, M], -1 padded
    seq_lens: np.ndarray            # int32 [B]
    query_lens: np.ndarray          # int32 [B]
    query_start_loc: np.ndarray     # int32 [B+1]
    positions: np.ndarray           # int32 [T], positions of the new tokens
    query: np.ndarray               # [T, Hq, D]  (uint16 bits or float32)
    key: np.ndarray                 # [T, Hkv, D] new tokens
    value: np.ndarray               # [T, Hkv, D]
    key_cache: np.ndarray           # [NB, bs, Hkv, D] before the write
    value_cache: np.ndarray
    ref_counts: np.ndarray          # int32 [NB]
    is_prefill: np.ndarray          # bool [B]
    logical_k: Optional[List[np.ndarray]] = None   # per seq [seq_len, Hkv, D] incl. new tokens
    logical_v: Optional[List[np.ndarray]] = None

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.positions.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.query_lens.size else 0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.spec.dtype == "f32" else 2

    def kv_bytes_logical(self) -> int:
        """KV bytes one attention pass must read: each sequence's K and V once
        per KV head (shared prefix counted once per sharer)."""
        s = self.spec
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * s.num_kv_heads * s.head_dim * self.elem_bytes

    def kv_bytes_unique(self) -> int:
        """KV bytes of the physically distinct tokens attended (shared prefix once)."""
        s = self.spec
        total = int(self.seq_lens.astype(np.int64).sum())
        if s.shared_prefix_tokens and self.num_seqs > 1:
            total -= (self.num_seqs - 1) * s.shared_prefix_tokens
        return total * 2 * s.num_kv_heads * s.head_dim * self.elem_bytes


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return _to_bf16_bits(x) if dtype == "bf16" else x


def _draw_lengths(rng: np.random.Generator, kind: Tuple, n: int) -> np.ndarray:
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    tag = kind[0]
    if tag == "fixed":
        vals = np.asarray(kind[1], dtype=np.int64)
        if vals.shape[0] != n:
            raise ValueError("fixed lengths need %d values" % n)
        return vals
    if tag == "uniform":
        return rng.integers(kind[1], kind[2], size=n, endpoint=True).astype(np.int64)
    if tag == "lognormal":
        median, sigma, lo, hi = kind[1:]
        x = rng.normal(math.log(median), sigma, size=n)
        return np.clip(np.rint(np.exp(x)), lo, hi).astype(np.int64)
    raise ValueError("unknown length kind %r" % (tag,))


def generate(cfg, seed: Optional[int] = None, keep_logical: bool = False) -> Workload:
    """Build the workload for config ``cfg`` (an index into CONFIGS or a spec)."""
    spec = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    seed = spec.default_seed if seed is None else int(seed)
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")

    # 1. lengths: (ctx, q) per sequence
    dec = _draw_lengths(rng, spec.decode_len, spec.num_decode)
    dec_ctx = dec if spec.decode_len_is_ctx else dec - 1
    pre_ctx = _draw_lengths(rng, spec.prefill_ctx, spec.num_prefill)
    chunks = spec.prefill_chunk if isinstance(spec.prefill_chunk, tuple) else (spec.prefill_chunk,) * spec.num_prefill
    if len(chunks) != spec.num_prefill:
        raise ValueError("prefill_chunk needs one length per prefill")
    pre = [(int(c), int(q), True) for c, q in zip(pre_ctx, chunks)]
    dcd = [(int(c), 1, False) for c in dec_ctx]
    seqs = pre + dcd if spec.prefill_first else dcd + pre
    B = len(seqs)
    ctx = np.array([s[0] for s in seqs], dtype=np.int64)
    qlen = np.array([s[1] for s in seqs], dtype=np.int64)
    seq_lens = ctx + qlen
    is_prefill = np.array([s[2] for s in seqs], dtype=bool)
    share = spec.shared_prefix_tokens
    if share:
        if share % bs or np.any(ctx < share):
            raise ValueError("shared prefix must be block aligned and cached in every sequence")
        if np.any(is_prefill):
            raise ValueError("shared prefix workloads are decode-only")

    # 2. pool and placement
    nblk = -(-seq_lens // bs)
    unique_blocks = int(nblk.sum()) - (B - 1) * (share // bs if B else 0)
    NB = spec.pool_blocks if spec.pool_blocks is not None else int(math.ceil(spec.pool_slack * unique_blocks))
    if NB < unique_blocks:
        raise ValueError("pool of %d blocks cannot hold %d" % (NB, unique_blocks))
    pool = BlockPool(NB, order=rng.permutation(NB))
    tables: List[SeqBlocks] = []
    for s in range(B):
        t = SeqBlocks(bs)
        if share and s > 0:
            t.share_prefix_from(tables[0], share // bs, pool)
            t.append_tokens(int(seq_lens[s]) - share, pool)
        else:
            t.append_tokens(int(seq_lens[s]), pool)
        tables.append(t)
    block_tables = np.array(tables_to_rows(tables), dtype=np.int32)

    # 3. query
    T = int(qlen.sum())
    query = _draw_values(rng, (T, Hq, D), spec.dtype)

    # 4. cached K, then cached V, per physically distinct cached token
    kind = np.uint16 if spec.dtype == "bf16" else np.float32
    nan_bits = BF16_NAN if spec.dtype == "bf16" else F32_NAN_BITS.view(np.float32)
    pools = []
    for _which in range(2):
        cache = np.full((NB, bs, Hkv, D), nan_bits, dtype=kind)
        per_seq = []
        for s in range(B):
            first = share if (share and s > 0) else 0
            rows = _draw_values(rng, (int(ctx[s]) - first, Hkv, D), spec.dtype)
            per_seq.append(rows)
            for lb in range(first // bs, -(-int(ctx[s]) // bs)):
                lo = lb * bs
                n = min(bs, int(ctx[s]) - lo)
                cache[tables[s].mapping[lb], :n] = rows[lo - first: lo - first + n]
        pools.append((cache, per_seq))
    (key_cache, k_rows), (value_cache, v_rows) = pools

    # 5. the step's new tokens
    key = _draw_values(rng, (T, Hkv, D), spec.dtype)
    value = _draw_values(rng, (T, Hkv, D), spec.dtype)

    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(qlen)
    positions = np.concatenate([np.arange(ctx[s], ctx[s] + qlen[s]) for s in range(B)]).astype(np.int32) \
        if B else np.zeros(0, dtype=np.int32)

    wl = Workload(
        spec=spec, seed=seed, scale=1.0 / math.sqrt(D), num_blocks=NB,
        block_tables=block_tables, seq_lens=seq_lens.astype(np.int32), query_lens=qlen.astype(np.int32),
        query_start_loc=qsl, positions=positions, query=query, key=key, value=value,
        key_cache=key_cache, value_cache=value_cache,
        ref_counts=np.array(pool.ref_counts(), dtype=np.int32), is_prefill=is_prefill)

    if keep_logical:
        lk, lv = [], []
        for s in range(B):
            parts_k, parts_v = [], []
            if share and s > 0:
                parts_k.append(k_rows[0][:share])
                parts_v.append(v_rows[0][:share])
            parts_k += [k_rows[s], key[qsl[s]:qsl[s + 1]]]
            parts_v += [v_rows[s], value[qsl[s]:qsl[s + 1]]]
            lk.append(np.concatenate(parts_k, axis=0))
            lv.append(np.concatenate(parts_v, axis=0))
        wl.logical_k, wl.logical_v = lk, lv
    return wl


def reduced(cfg: int, **overrides) -> WorkloadSpec:
    """A smaller variant of a config (same structure), for fast parity runs."""
    return CONFIGS[cfg].with_(**overrides)


# ---------------------------------------------------------------- request streams
class TokenBank:
    """Synthetic query/key/value rows for any (request, position): a bank of
    `size` seeded rows, and token p of request r reads row
    (r * 1000003 + p * 7919) mod size.  The values depend only on (seed, r,
    p), so a token recomputed after a preemption gets the same K/V, and a
    step's inputs are a gather from the bank (no per-token generation)."""

    def __init__(self, seed: int, size: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 dtype: str = "bf16"):
        rng = np.random.default_rng([int(seed), 99])
        self.size = int(size)
        self.q = _draw_values(rng, (self.size, num_q_heads, head_dim), dtype)
        self.k = _draw_values(rng, (self.size, num_kv_heads, head_dim), dtype)
        self.v = _draw_values(rng, (self.size, num_kv_heads, head_dim), dtype)

    def index(self, req_id, positions) -> np.ndarray:
        """Bank rows of tokens (req_id may be a scalar or one id per position)."""
        p = np.asarray(positions, dtype=np.int64)
        return (np.asarray(req_id, dtype=np.int64) * 1000003 + p * 7919) % self.size

    def rows(self, req_id: int, positions):
        i = self.index(req_id, positions)
        return self.q[i], self.k[i], self.v[i]


def request_mix(seed: int, n: int, prompt=("lognormal", 300.0, LOGNORMAL_SIGMA, 8, 2048),
                new_tokens=("uniform", 8, 64), arrivals_per_step: float = 0.0):
    """n requests as (req_id, prompt_len, max_new_tokens, arrival_step): prompt
    lengths from `prompt`, generation lengths from `new_tokens`; arrivals
    all at step 0, or Poisson with the given mean per step."""
    rng = np.random.default_rng([int(seed), 7])
    p = _draw_lengths(rng, prompt, n)
    g = _draw_lengths(rng, new_tokens, n)
    if arrivals_per_step > 0:
        gaps = rng.poisson(1.0 / arrivals_per_step, n) if arrivals_per_step < 1 else np.zeros(n, np.int64)
        arr = np.cumsum(gaps)
        if arrivals_per_step >= 1:
            arr = np.arange(n) // int(arrivals_per_step)
    else:
        arr = np.zeros(n, np.int64)
    return [(i, int(p[i]), int(g[i]), int(arr[i])) for i in range(n)]
