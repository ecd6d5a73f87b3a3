"""Python binding of libpagedkv.so (argument marshalling only).

Every function takes torch tensors that already live on the GPU, checks their
dtype/shape/contiguity, and passes raw device pointers plus the current HIP
stream to the C ABI declared in include/pagedkv.h.  All compute happens in the
library's HIP kernels; there is no CPU path.  A missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
_c_i32, _c_i64, _c_f32, _c_sz, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "pkv_version": (_c_i32, []),
    "pkv_status_string": (ctypes.c_char_p, [_c_i32]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_compute_slot_mapping": (_c_i32, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp]),
    "pkv_reshape_and_cache": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i64,
                                       _c_i32, _c_i32, _c_vp]),
    "pkv_write_new_tokens": (_c_i32, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp,
                                      _c_vp, _c_i32, _c_i32, _c_i64, _c_i32, _c_vp, _c_vp]),
    "pkv_decode_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pkv_paged_attention_decode": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32, _c_i32,
                                            _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_f32, _c_i32, _c_vp,
                                            _c_sz, _c_vp]),
    "pkv_varlen_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pkv_paged_attention_varlen": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,
                                            _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                                            _c_f32, _c_i32, _c_vp, _c_sz, _c_vp]),
    "pkv_reshape_and_cache_fp8": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i64,
                                           _c_i32, _c_i32, _c_f32, _c_f32, _c_vp]),
    "pkv_write_new_tokens_fp8": (_c_i32, [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp,
                                          _c_vp, _c_i32, _c_i32, _c_i64, _c_i32, _c_f32, _c_f32, _c_vp, _c_vp]),
    "pkv_paged_attention_decode_fp8": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32, _c_i32,
                                                _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_f32, _c_f32, _c_f32,
                                                _c_vp, _c_sz, _c_vp]),
    "pkv_paged_attention_varlen_fp8": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,
                                                _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                                                _c_f32, _c_f32, _c_f32, _c_vp, _c_sz, _c_vp]),
    "pkv_decode_step": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32, _c_i32,
                                 _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_f32, _c_i32, _c_vp, _c_sz, _c_vp]),
    "pkv_decode_step_fp8": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32,
                                     _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_f32, _c_f32, _c_f32, _c_vp,
                                     _c_sz, _c_vp]),
    "pkv_decode_shared_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pkv_paged_attention_decode_shared": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32, _c_i32,
                                                   _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_f32, _c_i32, _c_vp,
                                                   _c_i32, _c_vp, _c_sz, _c_vp]),
    "pkv_paged_attention_decode_shared_fp8": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32,
                                                       _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_f32, _c_f32,
                                                       _c_f32, _c_vp, _c_i32, _c_vp, _c_sz, _c_vp]),
    "pkv_decode_step_shared": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32,
                                        _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_f32, _c_i32, _c_vp, _c_i32,
                                        _c_vp, _c_sz, _c_vp]),
    "pkv_paged_attention_decode_noalloc": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32,
                                                    _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_f32, _c_i32,
                                                    _c_vp]),
    "pkv_noalloc_scratch_bytes": (_c_sz, []),
    "pkv_sched_create": (_c_vp, [_c_vp, _c_vp]),
    "pkv_sched_destroy": (None, [_c_vp]),
    "pkv_sched_add_request": (_c_i32, [_c_vp, _c_i64, _c_i32, _c_i32]),
    "pkv_sched_has_work": (_c_i32, [_c_vp]),
    "pkv_sched_schedule": (_c_i32, [_c_vp, _c_vp]),
    "pkv_sched_complete": (_c_i32, [_c_vp]),
    "pkv_sched_num_free_gpu": (_c_i32, [_c_vp]),
    "pkv_sched_num_free_cpu": (_c_i32, [_c_vp]),
    "pkv_sched_count": (_c_i32, [_c_vp, _c_i32]),
    "pkv_sched_request_info": (_c_i32, [_c_vp, _c_i64, _c_vp, _c_vp, _c_vp]),
    "pkv_copy_blocks": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_vp]),
    "pkv_swap_blocks": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_vp]),
    "pkv_set_profile_events": (_c_i32, [_c_vp, _c_vp]),
    "pkv_stream_read": (_c_i32, [_c_vp, _c_sz, _c_vp, _c_i32, _c_vp]),
    "pkv_set_decode_workers": (_c_i32, [_c_i32]),
    "pkv_set_waves_per_cu": (_c_i32, [_c_i32]),
    "pkv_set_decode_segment_cost": (_c_i32, [_c_i32]),
    "pkv_set_decode_dynamic": (_c_i32, [_c_i32, _c_i32]),
    "pkv_set_varlen_single_launch": (_c_i32, [_c_i32]),
    "pkv_get_waves_per_cu": (_c_i32, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libpagedkv.so, building it first only if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build_lib
            build_lib.build()
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


class PagedKVError(RuntimeError):
    pass


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise PagedKVError("%s failed: %s (%s)" % (what, L.pkv_status_string(status).decode(),
                                                   L.pkv_last_error().decode()))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %d" % (name, ndim, t.dim()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise ValueError("KV dtype must be bfloat16 or float32, got %s" % t.dtype)


# ----------------------------------------------------------------- the four calls
def compute_slot_mapping(block_tables: torch.Tensor, positions: torch.Tensor, query_start_loc: torch.Tensor,
                         block_size: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """slot[t] = block_tables[s][pos // bs] * bs + pos % bs (int64, -1 for padding)."""
    B, M = block_tables.shape
    T = positions.shape[0]
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=positions.device)
    if query_start_loc.shape[0] != B + 1:
        raise ValueError("query_start_loc must have num_seqs + 1 entries")
    _check(lib().pkv_compute_slot_mapping(_dev(block_tables, "block_tables", torch.int32, 2), B, M,
                                          _dev(positions, "positions", torch.int32, 1),
                                          _dev(query_start_loc, "query_start_loc", torch.int32, 1), T,
                                          int(block_size), _dev(out, "slot_mapping", torch.int64, 1),
                                          _stream(positions)), "compute_slot_mapping")
    return out


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                      slot_mapping: torch.Tensor) -> None:
    """Scatter key/value [T, Hkv, D] rows into the [NB, bs, Hkv, D] pools at their slots."""
    T, Hkv, D = key.shape
    NB, bs = key_cache.shape[0], key_cache.shape[1]
    if value.shape != key.shape or value_cache.shape != key_cache.shape or key_cache.shape[2:] != (Hkv, D):
        raise ValueError("key/value/cache shapes disagree")
    if key.dtype != key_cache.dtype or value.dtype != key.dtype or value_cache.dtype != key.dtype:
        raise ValueError("key/value/caches must share one dtype")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one entry per token")
    _check(lib().pkv_reshape_and_cache(_dev(key, "key", ndim=3), _dev(value, "value", ndim=3),
                                       _dev(key_cache, "key_cache", ndim=4), _dev(value_cache, "value_cache", ndim=4),
                                       _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, Hkv, D, NB, bs,
                                       _kv_dtype(key), _stream(key)), "reshape_and_cache")


def write_new_tokens(block_tables: torch.Tensor, positions: torch.Tensor, query_start_loc: torch.Tensor,
                     block_size: int, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                     value_cache: torch.Tensor, slot_mapping: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """compute_slot_mapping + reshape_and_cache in one kernel; returns the
    slots if ``slot_mapping`` is given (written in place)."""
    B, M = block_tables.shape
    T, Hkv, D = key.shape
    NB, bs = key_cache.shape[0], key_cache.shape[1]
    if value.shape != key.shape or value_cache.shape != key_cache.shape or key_cache.shape[2:] != (Hkv, D):
        raise ValueError("key/value/cache shapes disagree")
    if key.dtype != key_cache.dtype or value.dtype != key.dtype or value_cache.dtype != key.dtype:
        raise ValueError("key/value/caches must share one dtype")
    if positions.shape[0] != T or query_start_loc.shape[0] != B + 1 or bs != block_size:
        raise ValueError("positions/query_start_loc/block_size do not match")
    sp = _dev(slot_mapping, "slot_mapping", torch.int64, 1) if slot_mapping is not None else None
    _check(lib().pkv_write_new_tokens(_dev(block_tables, "block_tables", torch.int32, 2), B, M,
                                      _dev(positions, "positions", torch.int32, 1),
                                      _dev(query_start_loc, "query_start_loc", torch.int32, 1), T, int(block_size),
                                      _dev(key, "key", ndim=3), _dev(value, "value", ndim=3),
                                      _dev(key_cache, "key_cache", ndim=4), _dev(value_cache, "value_cache", ndim=4),
                                      Hkv, D, NB, _kv_dtype(key), sp, _stream(key)), "write_new_tokens")
    return slot_mapping


def decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                          dtype: torch.dtype) -> int:
    return int(lib().pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                               PKV_BF16 if dtype == torch.bfloat16 else PKV_F32))


def varlen_workspace_size(num_seqs: int, num_tokens: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          max_query_len: int, block_size: int, dtype: torch.dtype) -> int:
    return int(lib().pkv_varlen_workspace_size(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                               max_query_len, block_size,
                                               PKV_BF16 if dtype == torch.bfloat16 else PKV_F32))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    # the library checks the size (PKV_EWORKSPACE); this only allocates a
    # default, zero-filled as a new workspace must be
    if workspace is None:
        return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
    return workspace


def paged_attention_decode(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                           block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, max_seq_len: int,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[s, h] = softmax(scale * q[s, h] K^T) V over seq_lens[s] paged tokens; float32 [B, Hq, D]."""
    B, Hq, D = query.shape
    NB, bs, Hkv, Dk = key_cache.shape
    if Dk != D or value_cache.shape != key_cache.shape:
        raise ValueError("cache shapes disagree with the query")
    if query.dtype != key_cache.dtype or value_cache.dtype != key_cache.dtype:
        raise ValueError("query and caches must share one dtype")
    if block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_tables/seq_lens must have num_seqs rows")
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=query.device)
    ws = _workspace(decode_workspace_size(B, Hq, Hkv, D, bs, query.dtype), query.device, workspace)
    _check(lib().pkv_paged_attention_decode(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key_cache, "key_cache", ndim=4),
        _dev(value_cache, "value_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32, 2),
        block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1), B, Hq, Hkv, D, NB, bs,
        int(max_seq_len), float(scale), _kv_dtype(query), _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), _stream(query)), "paged_attention_decode")
    return out


def paged_attention_decode_noalloc(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                                   block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, max_seq_len: int,
                                   out: torch.Tensor) -> torch.Tensor:
    """paged_attention_decode without a workspace: the library's allocation-free
    entry point, whose split-K scratch is a static device array.  `out`
    (float32 [B, Hq, D]) is required, so nothing is allocated on this path."""
    B, Hq, D = query.shape
    NB, bs, Hkv, Dk = key_cache.shape
    if Dk != D or value_cache.shape != key_cache.shape:
        raise ValueError("cache shapes disagree with the query")
    if query.dtype != key_cache.dtype or value_cache.dtype != key_cache.dtype:
        raise ValueError("query and caches must share one dtype")
    if block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_tables/seq_lens must have num_seqs rows")
    _check(lib().pkv_paged_attention_decode_noalloc(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key_cache, "key_cache", ndim=4),
        _dev(value_cache, "value_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32, 2),
        block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1), B, Hq, Hkv, D, NB, bs,
        int(max_seq_len), float(scale), _kv_dtype(query), _stream(query)), "paged_attention_decode_noalloc")
    return out


def _groups(prefix_groups: torch.Tensor):
    g = prefix_groups
    if g.dim() != 2 or g.shape[1] != 3:
        raise ValueError("prefix_groups must be int32 [num_groups, 3]")
    return _dev(g, "prefix_groups", torch.int32, 2), int(g.shape[0])


def decode_shared_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                 block_size: int, dtype, num_groups: int) -> int:
    kind = PKV_FP8_E4M3 if dtype == torch.uint8 else (PKV_BF16 if dtype == torch.bfloat16 else PKV_F32)
    return int(lib().pkv_decode_shared_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                      kind, num_groups))


def paged_attention_decode_shared(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                                  block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                                  max_seq_len: int, prefix_groups: torch.Tensor, out: Optional[torch.Tensor] = None,
                                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """paged_attention_decode where prefix_groups (int32 [G, 3]: first sequence,
    sequences, shared tokens) names sequences whose first tokens live in the
    same blocks; each group's shared blocks are read once."""
    B, Hq, D = query.shape
    NB, bs, Hkv, Dk = key_cache.shape
    if Dk != D or value_cache.shape != key_cache.shape or query.dtype != key_cache.dtype:
        raise ValueError("cache shapes or dtypes disagree with the query")
    gp, ng = _groups(prefix_groups)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=query.device)
    ws = _workspace(decode_shared_workspace_size(B, Hq, Hkv, D, bs, query.dtype, ng), query.device, workspace)
    _check(lib().pkv_paged_attention_decode_shared(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key_cache, "key_cache", ndim=4),
        _dev(value_cache, "value_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32, 2),
        block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1), B, Hq, Hkv, D, NB, bs,
        int(max_seq_len), float(scale), _kv_dtype(query), gp, ng, _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), _stream(query)), "paged_attention_decode_shared")
    return out


def paged_attention_decode_shared_fp8(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                                      block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                                      max_seq_len: int, k_scale: float, v_scale: float, prefix_groups: torch.Tensor,
                                      out: Optional[torch.Tensor] = None,
                                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """paged_attention_decode_fp8 with shared-prefix groups (bf16 query, E4M3 pools)."""
    B, Hq, D = query.shape
    NB, bs, Hkv, Dk = key_cache.shape
    if key_cache.dtype != torch.uint8 or query.dtype != torch.bfloat16 or Dk != D:
        raise ValueError("E4M3 pools (uint8) and a bfloat16 query are required")
    gp, ng = _groups(prefix_groups)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=query.device)
    ws = _workspace(decode_shared_workspace_size(B, Hq, Hkv, D, bs, torch.uint8, ng), query.device, workspace)
    _check(lib().pkv_paged_attention_decode_shared_fp8(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key_cache, "key_cache", ndim=4),
        _dev(value_cache, "value_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32, 2),
        block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1), B, Hq, Hkv, D, NB, bs,
        int(max_seq_len), float(scale), float(k_scale), float(v_scale), gp, ng, _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), _stream(query)), "paged_attention_decode_shared_fp8")
    return out


def decode_step_shared(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                       max_seq_len: int, prefix_groups: torch.Tensor, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_step with shared-prefix groups: each sequence's new token is
    written to its slot, then attention reads each group's shared blocks once."""
    B, Hq, D = query.shape
    NB, bs, Hkv, Dk = key_cache.shape
    if Dk != D or value_cache.shape != key_cache.shape or query.dtype != key_cache.dtype:
        raise ValueError("cache shapes or dtypes disagree with the query")
    if key.shape != (B, Hkv, D) or value.shape != (B, Hkv, D):
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
    gp, ng = _groups(prefix_groups)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=query.device)
    ws = _workspace(decode_shared_workspace_size(B, Hq, Hkv, D, bs, query.dtype, ng), query.device, workspace)
    _check(lib().pkv_decode_step_shared(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key, "key", ndim=3),
        _dev(value, "value", ndim=3), _dev(key_cache, "key_cache", ndim=4), _dev(value_cache, "value_cache", ndim=4),
        _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
        _dev(seq_lens, "seq_lens", torch.int32, 1), B, Hq, Hkv, D, NB, bs, int(max_seq_len), float(scale),
        _kv_dtype(query), gp, ng, _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream(query)),
        "decode_step_shared")
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib().pkv_noalloc_scratch_bytes())


def paged_attention_varlen(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                           block_tables: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                           scale: float, max_query_len: int, max_seq_len: int, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mixed prefill-chunk + decode rows; float32 [T, Hq, D] (bottom-right causal)."""
    T, Hq, D = query.shape
    NB, bs, Hkv, Dk = key_cache.shape
    B = seq_lens.shape[0]
    if Dk != D or value_cache.shape != key_cache.shape:
        raise ValueError("cache shapes disagree with the query")
    if query.dtype != key_cache.dtype or value_cache.dtype != key_cache.dtype:
        raise ValueError("query and caches must share one dtype")
    if block_tables.shape[0] != B or query_start_loc.shape[0] != B + 1:
        raise ValueError("block_tables/query_start_loc do not match seq_lens")
    if out is None:
        out = torch.empty(T, Hq, D, dtype=torch.float32, device=query.device)
    ws = _workspace(varlen_workspace_size(B, T, Hq, Hkv, D, max_query_len, bs, query.dtype), query.device, workspace)
    _check(lib().pkv_paged_attention_varlen(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key_cache, "key_cache", ndim=4),
        _dev(value_cache, "value_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32, 2),
        block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1),
        _dev(query_start_loc, "query_start_loc", torch.int32, 1), B, T, int(max_query_len), int(max_seq_len),
        Hq, Hkv, D, NB, bs, float(scale), _kv_dtype(query), _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), _stream(query)), "paged_attention_varlen")
    return out


# ----------------------------------------------------------------- FP8 (E4M3) pools
_FP8_POOL = (torch.uint8, torch.float8_e4m3fn)


def _fp8_pools(key_cache: torch.Tensor, value_cache: torch.Tensor) -> None:
    if key_cache.dtype not in _FP8_POOL or value_cache.dtype not in _FP8_POOL:
        raise ValueError("E4M3 pools must be uint8 or float8_e4m3fn tensors")
    if value_cache.shape != key_cache.shape:
        raise ValueError("key_cache and value_cache shapes differ")


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                          value_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float,
                          v_scale: float) -> None:
    """reshape_and_cache into E4M3 pools: code = E4M3(x * (1/scale)), saturating."""
    T, Hkv, D = key.shape
    _fp8_pools(key_cache, value_cache)
    NB, bs = key_cache.shape[0], key_cache.shape[1]
    if value.shape != key.shape or key_cache.shape[2:] != (Hkv, D) or value.dtype != key.dtype:
        raise ValueError("key/value/cache shapes disagree")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one entry per token")
    _check(lib().pkv_reshape_and_cache_fp8(_dev(key, "key", ndim=3), _dev(value, "value", ndim=3),
                                           _dev(key_cache, "key_cache", ndim=4),
                                           _dev(value_cache, "value_cache", ndim=4),
                                           _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, Hkv, D, NB, bs,
                                           _kv_dtype(key), float(k_scale), float(v_scale), _stream(key)),
           "reshape_and_cache_fp8")


def write_new_tokens_fp8(block_tables: torch.Tensor, positions: torch.Tensor, query_start_loc: torch.Tensor,
                         block_size: int, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, k_scale: float, v_scale: float,
                         slot_mapping: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """write_new_tokens into E4M3 pools (slot mapping + quantising write)."""
    B, M = block_tables.shape
    T, Hkv, D = key.shape
    _fp8_pools(key_cache, value_cache)
    NB, bs = key_cache.shape[0], key_cache.shape[1]
    if value.shape != key.shape or key_cache.shape[2:] != (Hkv, D) or value.dtype != key.dtype:
        raise ValueError("key/value/cache shapes disagree")
    if positions.shape[0] != T or query_start_loc.shape[0] != B + 1 or bs != block_size:
        raise ValueError("positions/query_start_loc/block_size do not match")
    sp = _dev(slot_mapping, "slot_mapping", torch.int64, 1) if slot_mapping is not None else None
    _check(lib().pkv_write_new_tokens_fp8(_dev(block_tables, "block_tables", torch.int32, 2), B, M,
                                          _dev(positions, "positions", torch.int32, 1),
                                          _dev(query_start_loc, "query_start_loc", torch.int32, 1), T,
                                          int(block_size), _dev(key, "key", ndim=3), _dev(value, "value", ndim=3),
                                          _dev(key_cache, "key_cache", ndim=4),
                                          _dev(value_cache, "value_cache", ndim=4), Hkv, D, NB, _kv_dtype(key),
                                          float(k_scale), float(v_scale), sp, _stream(key)), "write_new_tokens_fp8")
    return slot_mapping


def paged_attention_decode_fp8(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                               block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, max_seq_len: int,
                               k_scale: float, v_scale: float, out: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention over E4M3 pools (K = code * k_scale, V = code * v_scale); bf16 query."""
    B, Hq, D = query.shape
    _fp8_pools(key_cache, value_cache)
    NB, bs, Hkv, Dk = key_cache.shape
    if Dk != D or query.dtype != torch.bfloat16:
        raise ValueError("query must be bfloat16 [B, Hq, D] matching the pools")
    if block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_tables/seq_lens must have num_seqs rows")
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=query.device)
    nbytes = int(lib().pkv_decode_workspace_size(B, Hq, Hkv, D, bs, PKV_FP8_E4M3))
    ws = _workspace(nbytes, query.device, workspace)
    _check(lib().pkv_paged_attention_decode_fp8(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key_cache, "key_cache", ndim=4),
        _dev(value_cache, "value_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32, 2),
        block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1), B, Hq, Hkv, D, NB, bs,
        int(max_seq_len), float(scale), float(k_scale), float(v_scale), _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), _stream(query)), "paged_attention_decode_fp8")
    return out


def _step_rows(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor) -> None:
    B, Hq, D = query.shape
    if key.shape != (B, key_cache.shape[2], D) or value.shape != key.shape:
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise ValueError("key/value must have the query's dtype")


def decode_step(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                value_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                max_seq_len: int, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step: write each sequence's new token (position seq_lens[s]-1,
    rows key[s]/value[s]) into its slot, then decode attention; float32 [B, Hq, D]."""
    B, Hq, D = query.shape
    NB, bs, Hkv, Dk = key_cache.shape
    if Dk != D or value_cache.shape != key_cache.shape:
        raise ValueError("cache shapes disagree with the query")
    if query.dtype != key_cache.dtype or value_cache.dtype != key_cache.dtype:
        raise ValueError("query and caches must share one dtype")
    if block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_tables/seq_lens must have num_seqs rows")
    _step_rows(query, key, value, key_cache)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=query.device)
    ws = _workspace(decode_workspace_size(B, Hq, Hkv, D, bs, query.dtype), query.device, workspace)
    _check(lib().pkv_decode_step(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key, "key", ndim=3),
        _dev(value, "value", ndim=3), _dev(key_cache, "key_cache", ndim=4), _dev(value_cache, "value_cache", ndim=4),
        _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
        _dev(seq_lens, "seq_lens", torch.int32, 1), B, Hq, Hkv, D, NB, bs, int(max_seq_len), float(scale),
        _kv_dtype(query), _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream(query)), "decode_step")
    return out


def decode_step_fp8(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                    value_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                    max_seq_len: int, k_scale: float, v_scale: float, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_step over E4M3 pools: bf16 query/key/value, quantising write, E4M3 attention."""
    B, Hq, D = query.shape
    _fp8_pools(key_cache, value_cache)
    NB, bs, Hkv, Dk = key_cache.shape
    if Dk != D or query.dtype != torch.bfloat16:
        raise ValueError("query must be bfloat16 [B, Hq, D] matching the pools")
    if block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_tables/seq_lens must have num_seqs rows")
    _step_rows(query, key, value, key_cache)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=query.device)
    nbytes = int(lib().pkv_decode_workspace_size(B, Hq, Hkv, D, bs, PKV_FP8_E4M3))
    ws = _workspace(nbytes, query.device, workspace)
    _check(lib().pkv_decode_step_fp8(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key, "key", ndim=3),
        _dev(value, "value", ndim=3), _dev(key_cache, "key_cache", ndim=4), _dev(value_cache, "value_cache", ndim=4),
        _dev(block_tables, "block_tables", torch.int32, 2), block_tables.shape[1],
        _dev(seq_lens, "seq_lens", torch.int32, 1), B, Hq, Hkv, D, NB, bs, int(max_seq_len), float(scale),
        float(k_scale), float(v_scale), _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream(query)),
        "decode_step_fp8")
    return out


def paged_attention_varlen_fp8(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                               block_tables: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                               scale: float, max_query_len: int, max_seq_len: int, k_scale: float, v_scale: float,
                               out: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Varlen attention over E4M3 pools; bf16 query."""
    T, Hq, D = query.shape
    _fp8_pools(key_cache, value_cache)
    NB, bs, Hkv, Dk = key_cache.shape
    B = seq_lens.shape[0]
    if Dk != D or query.dtype != torch.bfloat16:
        raise ValueError("query must be bfloat16 [T, Hq, D] matching the pools")
    if block_tables.shape[0] != B or query_start_loc.shape[0] != B + 1:
        raise ValueError("block_tables/query_start_loc do not match seq_lens")
    if out is None:
        out = torch.empty(T, Hq, D, dtype=torch.float32, device=query.device)
    nbytes = int(lib().pkv_varlen_workspace_size(B, T, Hq, Hkv, D, max_query_len, bs, PKV_FP8_E4M3))
    ws = _workspace(nbytes, query.device, workspace)
    _check(lib().pkv_paged_attention_varlen_fp8(
        _dev(out, "out", torch.float32, 3), _dev(query, "query", ndim=3), _dev(key_cache, "key_cache", ndim=4),
        _dev(value_cache, "value_cache", ndim=4), _dev(block_tables, "block_tables", torch.int32, 2),
        block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32, 1),
        _dev(query_start_loc, "query_start_loc", torch.int32, 1), B, T, int(max_query_len), int(max_seq_len),
        Hq, Hkv, D, NB, bs, float(scale), float(k_scale), float(v_scale), _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), _stream(query)), "paged_attention_varlen_fp8")
    return out


# ----------------------------------------------------------------- block copies
def _block_bytes(pool: torch.Tensor) -> int:
    return pool[0].numel() * pool.element_size() if pool.shape[0] else 0


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, block_mapping: torch.Tensor) -> None:
    """Copy-on-write copies: block dst of each pool becomes block src, for
    every (src, dst) row of the int64 [N, 2] mapping (on the GPU)."""
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("key_cache and value_cache must have one shape and dtype")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [N, 2]")
    _check(lib().pkv_copy_blocks(_dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
                                 _dev(block_mapping, "block_mapping", torch.int64, 2), block_mapping.shape[0],
                                 key_cache.shape[0], _block_bytes(key_cache), _stream(key_cache)), "copy_blocks")


def _pool_ptr(t: Optional[torch.Tensor], name: str) -> int:
    """A GPU tensor, or a pinned CPU tensor (the library maps it)."""
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous tensor" % name)
    if not t.is_cuda and not t.is_pinned():
        raise ValueError("%s must be on the GPU or in pinned host memory" % name)
    return t.data_ptr()


def swap_blocks(src_key: torch.Tensor, src_value: Optional[torch.Tensor], dst_key: torch.Tensor,
                dst_value: Optional[torch.Tensor], block_mapping: torch.Tensor, device=None) -> None:
    """Swap-out / swap-in: block dst of the dst pools becomes block src of the
    src pools for every (src, dst) row of block_mapping.  Pools are GPU or
    pinned CPU tensors with equal block shapes; the copy runs on ``device``
    (the GPU side's device by default) on its current stream."""
    pools = [p for p in (src_key, src_value, dst_key, dst_value) if p is not None]
    if any(p.shape[1:] != src_key.shape[1:] or p.dtype != src_key.dtype for p in pools):
        raise ValueError("pools must share block shape and dtype")
    if (src_value is None) != (dst_value is None):
        raise ValueError("src_value and dst_value must be both given or both None")
    if src_value is not None and (src_value.shape != src_key.shape or dst_value.shape != dst_key.shape):
        raise ValueError("key and value pools of one side must match")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2 or block_mapping.dtype != torch.int64:
        raise ValueError("block_mapping must be int64 [N, 2]")
    if device is None:
        device = next((p.device for p in pools + [block_mapping] if p.is_cuda), None)
        if device is None:
            raise ValueError("no GPU tensor given: pass device")
    with torch.cuda.device(device):
        _check(lib().pkv_swap_blocks(_pool_ptr(src_key, "src_key"), _pool_ptr(src_value, "src_value"),
                                     _pool_ptr(dst_key, "dst_key"), _pool_ptr(dst_value, "dst_value"),
                                     _pool_ptr(block_mapping, "block_mapping"), block_mapping.shape[0],
                                     src_key.shape[0], dst_key.shape[0], _block_bytes(src_key),
                                     torch.cuda.current_stream(device).cuda_stream), "swap_blocks")


# ----------------------------------------------------------------- knobs and timing
def set_decode_workers(n: int) -> int:
    return int(lib().pkv_set_decode_workers(int(n)))


def set_decode_segment_cost(n: int) -> int:
    """Virtual chunks the decode split charges per (sequence, KV head) range;
    returns the previous value."""
    return int(lib().pkv_set_decode_segment_cost(int(n)))


def set_decode_dynamic(permille: int, unit_chunks: int = 4) -> int:
    """Share (permille) of the decode split handed out in units of at least
    unit_chunks chunks to the wavefronts that finish first (-1: chosen per
    call); returns the previous share."""
    return int(lib().pkv_set_decode_dynamic(int(permille), int(unit_chunks)))


def varlen_single_launch() -> bool:
    """The current setting of set_varlen_single_launch."""
    prev = set_varlen_single_launch(True)
    set_varlen_single_launch(prev)
    return prev


def set_varlen_single_launch(on: bool) -> bool:
    """Whether mixed varlen steps (bf16/E4M3 pools, head_dim 128) run prefill
    and decode rows in one launch; returns the previous setting."""
    r = int(lib().pkv_set_varlen_single_launch(1 if on else 0))
    if r < 0:
        raise PagedKVError("pkv_set_varlen_single_launch failed")
    return bool(r)


def set_waves_per_cu(n: int) -> int:
    return int(lib().pkv_set_waves_per_cu(int(n)))


class HipEvent:
    """A raw hipEvent_t (created through the HIP runtime torch already loaded)."""
    _rt = None

    @classmethod
    def _runtime(cls):
        if cls._rt is None:
            rt = ctypes.CDLL("libamdhip64.so")
            rt.hipEventCreate.argtypes = [ctypes.POINTER(_c_vp)]
            rt.hipEventDestroy.argtypes = [_c_vp]
            rt.hipEventSynchronize.argtypes = [_c_vp]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _c_vp, _c_vp]
            cls._rt = rt
        return cls._rt

    def __init__(self):
        h = _c_vp()
        if self._runtime().hipEventCreate(ctypes.byref(h)) != 0:
            raise PagedKVError("hipEventCreate failed")
        self.handle = h

    def __del__(self):
        try:
            if self._rt is not None and self.handle:
                self._rt.hipEventDestroy(self.handle)
        except Exception:
            pass

    @staticmethod
    def elapsed_ms(start: "HipEvent", stop: "HipEvent") -> float:
        rt = HipEvent._runtime()
        rt.hipEventSynchronize(stop.handle)
        ms = ctypes.c_float()
        if rt.hipEventElapsedTime(ctypes.byref(ms), start.handle, stop.handle) != 0:
            raise PagedKVError("hipEventElapsedTime failed")
        return float(ms.value)


def set_profile_events(start: Optional[HipEvent], stop: Optional[HipEvent]) -> None:
    _check(lib().pkv_set_profile_events(start.handle if start else None, stop.handle if stop else None),
           "set_profile_events")


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Enqueue a plain streaming read of buf's bytes (a measuring stick for the
    HBM read rate, or a read-only cache flush); sink (int32 holding the uint32
    words, length a multiple of 4) receives one XOR word per wavefront."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().pkv_stream_read(_dev(buf, "buf"), nbytes, _dev(sink, "sink", torch.int32, 1), sink.numel(),
                                 _stream(buf)), "stream_read")
