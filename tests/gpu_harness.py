"""Shared helpers for the GPU tests: upload a workload, run the HIP path
through the C ABI binding, and compare with the float64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from paged_kv_cache_97_amd import ops
from paged_kv_cache_97_amd import workloads as W

TOL = {"f32": (1e-5, 1e-6), "bf16": (2e-2, 5e-3)}   # (max abs, relative L2)

# Pool scales of the E4M3 tests: not powers of two, so the float32 reciprocal
# used by the quantising write matters.
K_SCALE, V_SCALE = 0.0125, 0.02


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray, dtype: str, dev) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(dev)


def upload(wl, dev) -> dict:
    d = wl.spec.dtype
    return dict(
        query=to_dev(wl.query, d, dev), key=to_dev(wl.key, d, dev), value=to_dev(wl.value, d, dev),
        key_cache=to_dev(wl.key_cache, d, dev), value_cache=to_dev(wl.value_cache, d, dev),
        block_tables=torch.from_numpy(wl.block_tables).to(dev), seq_lens=torch.from_numpy(wl.seq_lens).to(dev),
        positions=torch.from_numpy(wl.positions).to(dev),
        query_start_loc=torch.from_numpy(wl.query_start_loc).to(dev))


def run_step(wl, t: dict, decode: bool = True):
    """One pass of the hot path: slot mapping -> cache write -> attention."""
    slots = ops.compute_slot_mapping(t["block_tables"], t["positions"], t["query_start_loc"], wl.spec.block_size)
    ops.reshape_and_cache(t["key"], t["value"], t["key_cache"], t["value_cache"], slots)
    if decode:
        out = ops.paged_attention_decode(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                         t["seq_lens"], wl.scale, wl.max_seq_len)
    else:
        out = ops.paged_attention_varlen(t["query"], t["key_cache"], t["value_cache"], t["block_tables"],
                                         t["seq_lens"], t["query_start_loc"], wl.scale, wl.max_query_len,
                                         wl.max_seq_len)
    torch.cuda.synchronize()
    return slots, out


def oracle_step(wl, decode: bool = True):
    slots = oracle.slot_mapping(wl.block_tables, wl.positions, wl.query_start_loc, wl.spec.block_size,
                                wl.num_blocks)
    kc, vc = oracle.reshape_and_cache(wl.key, wl.value, wl.key_cache, wl.value_cache, slots, wl.ref_counts)
    if decode:
        out = oracle.decode_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.scale, wl.spec.dtype)
    else:
        out = oracle.varlen_attention(wl.query, kc, vc, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                      wl.scale, wl.spec.dtype)
    return slots, kc, vc, out


def attn_errors(got: torch.Tensor, ref: np.ndarray):
    g = got.detach().cpu().double().numpy()
    diff = g - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel, bool(np.isfinite(g).all())


def assert_attn_close(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "", rel_factor: float = 1.0) -> None:
    """Max abs error within the stated bar; relative L2 within the builder's
    self-check, times rel_factor for scores larger than at scale 1/sqrt(D)."""
    max_abs, rel, finite = attn_errors(got, ref)
    tol_abs, tol_rel = TOL[dtype]
    tol_rel *= rel_factor
    log("  %s max|err| %.3g (tol %.0e)  rel-L2 %.3g (tol %.0e)" % (what, max_abs, tol_abs, rel, tol_rel))
    assert finite, "non-finite output"
    assert max_abs <= tol_abs, "max abs error %g > %g" % (max_abs, tol_abs)
    assert rel <= tol_rel, "relative L2 error %g > %g" % (rel, tol_rel)


def same_bits(a: torch.Tensor, b: np.ndarray) -> bool:
    """Bitwise equality of a device tensor with a host array of the same layout."""
    bt = torch.from_numpy(np.ascontiguousarray(b))
    if b.dtype == np.uint16:
        bt = bt.view(torch.bfloat16)
    bt = bt.to(a.device)
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), bt.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), bt.view(torch.int32))
    return torch.equal(a, bt)


# ------------------------------------------------------------------ E4M3 pools
def fp8_pools(wl, ks=K_SCALE, vs=V_SCALE):
    """The workload's pools as E4M3 codes (oracle encoder); free slots hold
    the E4M3 NaN byte 0xFF, as a reused block would hold stale data."""
    nan = W.BF16_NAN if wl.spec.dtype == "bf16" else None
    out = []
    for cache, sc in ((wl.key_cache, ks), (wl.value_cache, vs)):
        if nan is not None:
            live = cache != nan
        else:
            live = ~np.isnan(cache)
        q = np.full(cache.shape, 0xFF, np.uint8)
        q[live] = oracle.quantize_kv(cache[live], wl.spec.dtype, sc)
        out.append(q)
    return out


def upload_fp8(wl, dev, ks=K_SCALE, vs=V_SCALE):
    kq, vq = fp8_pools(wl, ks, vs)
    d = wl.spec.dtype
    q = wl.query if d == "bf16" else W._to_bf16_bits(wl.query)
    return dict(query=to_dev(q, "bf16", dev), key=to_dev(wl.key, d, dev), value=to_dev(wl.value, d, dev),
                key_cache=torch.from_numpy(kq).to(dev), value_cache=torch.from_numpy(vq).to(dev),
                kq=kq, vq=vq, q_bits=q,
                block_tables=torch.from_numpy(wl.block_tables).to(dev),
                seq_lens=torch.from_numpy(wl.seq_lens).to(dev), positions=torch.from_numpy(wl.positions).to(dev),
                query_start_loc=torch.from_numpy(wl.query_start_loc).to(dev))


def oracle_fp8_step(wl, t, decode=True, ks=K_SCALE, vs=V_SCALE):
    slots = oracle.slot_mapping(wl.block_tables, wl.positions, wl.query_start_loc, wl.spec.block_size,
                                wl.num_blocks)
    kc, vc = oracle.reshape_and_cache_fp8(wl.key, wl.value, t["kq"], t["vq"], slots, ks, vs, wl.spec.dtype,
                                          wl.ref_counts)
    if decode:
        out = oracle.decode_attention(t["q_bits"], kc, vc, wl.block_tables, wl.seq_lens, wl.scale, "bf16", (ks, vs))
    else:
        out = oracle.varlen_attention(t["q_bits"], kc, vc, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                      wl.scale, "bf16", (ks, vs))
    return slots, kc, vc, out
