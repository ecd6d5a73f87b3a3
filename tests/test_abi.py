"""The C ABI library loads, exports every call include/pagedkv.h declares,
and rejects bad arguments on the host before any launch.  CPU only: no call
here reaches a kernel."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_97_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = ops.lib()
    names = _declared()
    assert "pkv_paged_attention_decode" in names and "pkv_sched_schedule" in names and len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert n in ops._SIGNATURES, "binding lacks " + n


def test_status_strings_and_version():
    lib = ops.lib()
    assert lib.pkv_version() >= 100
    for code, word in [(0, b"OK"), (1, b"EINVAL"), (2, b"EUNSUPPORTED"), (3, b"EWORKSPACE"), (4, b"EHIP")]:
        assert word in lib.pkv_status_string(code)


def _decode(lib, **kw):
    args = dict(out=1 << 20, query=1 << 20, kc=1 << 20, vc=1 << 20, bt=1 << 20, max_blocks=4, seq_lens=1 << 20,
                B=2, Hq=8, Hkv=2, D=128, NB=16, bs=16, max_len=64, scale=0.1, dtype=1, ws=1 << 20,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.pkv_paged_attention_decode(args["out"], args["query"], args["kc"], args["vc"], args["bt"],
                                          args["max_blocks"], args["seq_lens"], args["B"], args["Hq"],
                                          args["Hkv"], args["D"], args["NB"], args["bs"], args["max_len"],
                                          args["scale"], args["dtype"], args["ws"], args["ws_bytes"],
                                          args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), 2), (dict(bs=8), 2), (dict(dtype=7), 2), (dict(Hq=7), 1), (dict(Hkv=0), 1),
    (dict(out=None), 1), (dict(query=(1 << 20) + 2), 1), (dict(B=9000), 2), (dict(ws_bytes=10), 3),
    (dict(ws=None), 3), (dict(ws=(1 << 20) + 16), 1), (dict(scale=float("inf")), 1), (dict(NB=0), 1),
])
def test_decode_validation_runs_before_any_launch(kw, code):
    lib = ops.lib()
    assert _decode(lib, **kw) == code
    assert lib.pkv_last_error()


def test_empty_work_enqueues_nothing():
    lib = ops.lib()
    assert _decode(lib, B=0) == 0
    assert lib.pkv_compute_slot_mapping(None, 0, 0, None, None, 0, 16, None, None) == 0
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 0, 8, 128, 0, 16, 1, None) == 0
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 3, 8, 128, 0, 16, 1, None) == 1
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 3, 1, 4, 0, 16, 1, None) == 2


def test_fused_write_validation():
    lib = ops.lib()
    args = [None, 2, 4, None, None, 0, 16, None, None, None, None, 8, 128, 10, 1, None, None]
    assert lib.pkv_write_new_tokens(*args) == 0                   # no tokens: nothing enqueued
    args[5] = 3
    assert lib.pkv_write_new_tokens(*args) == 1                   # null pointers
    bad = list(args); bad[11] = 1; bad[12] = 4
    assert lib.pkv_write_new_tokens(*bad) == 2                    # 8-byte rows
    bad = list(args); bad[14] = 9
    assert lib.pkv_write_new_tokens(*bad) == 2                    # dtype


def test_workspace_size_rules():
    lib = ops.lib()
    assert lib.pkv_decode_workspace_size(128, 64, 8, 128, 16, 1) > 0
    assert lib.pkv_decode_workspace_size(128, 64, 8, 96, 16, 1) == 0
    assert lib.pkv_decode_workspace_size(9000, 64, 8, 128, 16, 1) == 0
    prev = lib.pkv_set_decode_workers(100)
    small = lib.pkv_decode_workspace_size(4, 8, 2, 128, 16, 1)
    lib.pkv_set_decode_workers(1000)
    big = lib.pkv_decode_workspace_size(4, 8, 2, 128, 16, 1)
    lib.pkv_set_decode_workers(prev)
    assert big > small
    assert lib.pkv_set_decode_workers(-5) == -1
    assert lib.pkv_set_waves_per_cu(5) == -1
    assert lib.pkv_set_profile_events(ctypes.c_void_p(1), None) == 1


def test_block_copy_validation():
    lib = ops.lib()
    assert lib.pkv_copy_blocks(None, None, None, 0, 10, 4096, None) == 0          # no pairs: nothing enqueued
    assert lib.pkv_copy_blocks(None, None, None, 2, 10, 4096, None) == 1          # null pointers
    assert lib.pkv_copy_blocks(None, None, None, -1, 10, 4096, None) == 1
    assert lib.pkv_copy_blocks(None, None, None, 2, 10, 4100, None) == 1          # not a multiple of 16
    assert lib.pkv_swap_blocks(None, None, None, None, None, 0, 4, 4, 4096, None) == 0
    assert lib.pkv_swap_blocks(None, None, None, None, None, 3, 4, 4, 4096, None) == 1
    assert lib.pkv_swap_blocks(ctypes.c_void_p(256), ctypes.c_void_p(512), ctypes.c_void_p(768), None,
                               ctypes.c_void_p(1024), 3, 4, 4, 4096, None) == 1   # one value pool only
    assert lib.pkv_swap_blocks(None, None, None, None, None, 3, 4, -4, 4096, None) == 1
    assert lib.pkv_last_error()


def test_fp8_validation_runs_before_any_launch():
    lib = ops.lib()
    nul = [None] * 5
    # reshape_and_cache_fp8: no tokens -> OK; bad scales / dtype / row size -> errors
    assert lib.pkv_reshape_and_cache_fp8(*nul, 0, 8, 128, 10, 16, 1, 0.5, 0.5, None) == 0
    assert lib.pkv_reshape_and_cache_fp8(*nul, 0, 8, 128, 10, 16, 1, 0.0, 0.5, None) == 1
    assert lib.pkv_reshape_and_cache_fp8(*nul, 0, 8, 128, 10, 16, 1, 0.5, float("inf"), None) == 1
    assert lib.pkv_reshape_and_cache_fp8(*nul, 0, 8, 128, 10, 16, 2, 0.5, 0.5, None) == 2
    assert lib.pkv_reshape_and_cache_fp8(*nul, 0, 1, 8, 10, 16, 1, 0.5, 0.5, None) == 2
    assert lib.pkv_reshape_and_cache_fp8(*nul, 3, 8, 128, 10, 16, 1, 0.5, 0.5, None) == 1
    args = [None, 2, 4, None, None, 0, 16, None, None, None, None, 8, 128, 10, 1, 0.5, 0.5, None, None]
    assert lib.pkv_write_new_tokens_fp8(*args) == 0
    bad = list(args); bad[15] = -1.0
    assert lib.pkv_write_new_tokens_fp8(*bad) == 1
    # decode: E4M3 pools through the plain call are refused; the fp8 call checks its scales
    assert _decode(lib, dtype=2) == 1
    assert lib.pkv_decode_workspace_size(128, 64, 8, 128, 16, 2) == lib.pkv_decode_workspace_size(128, 64, 8, 128, 16, 1)
    a = [ctypes.c_void_p(1 << 20)] * 5
    st = lib.pkv_paged_attention_decode_fp8(a[0], a[1], a[2], a[3], a[4], 4, ctypes.c_void_p(1 << 20), 2, 8, 2, 128,
                                            10, 16, 64, 0.1, float("nan"), 1.0, ctypes.c_void_p(1 << 20), 1 << 30,
                                            None)
    assert st == 1 and b"scale" in lib.pkv_last_error()


def _step(lib, fp8=False, **kw):
    args = dict(out=1 << 20, query=1 << 20, key=1 << 20, value=1 << 20, kc=1 << 20, vc=1 << 20, bt=1 << 20,
                max_blocks=4, seq_lens=1 << 20, B=2, Hq=8, Hkv=2, D=128, NB=16, bs=16, max_len=64, scale=0.1,
                dtype=1, k_scale=0.5, v_scale=0.25, ws=1 << 20, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    head = [args[k] for k in ("out", "query", "key", "value", "kc", "vc", "bt", "max_blocks", "seq_lens", "B", "Hq",
                              "Hkv", "D", "NB", "bs", "max_len", "scale")]
    tail = [args["ws"], args["ws_bytes"], args["stream"]]
    if fp8:
        return lib.pkv_decode_step_fp8(*head, args["k_scale"], args["v_scale"], *tail)
    return lib.pkv_decode_step(*head, args["dtype"], *tail)


@pytest.mark.parametrize("fp8,kw,code", [
    (False, dict(key=None), 1), (False, dict(value=None), 1), (False, dict(key=(1 << 20) + 8), 1),
    (False, dict(dtype=2), 1), (False, dict(D=96), 2), (False, dict(out=None), 1), (False, dict(ws_bytes=10), 3),
    (False, dict(B=0, key=None, value=None), 0),
    (True, dict(k_scale=0.0), 1), (True, dict(v_scale=float("nan")), 1), (True, dict(value=None), 1),
    (True, dict(Hq=7), 1), (True, dict(B=0), 0),
])
def test_decode_step_validation_runs_before_any_launch(fp8, kw, code):
    lib = ops.lib()
    assert _step(lib, fp8, **kw) == code
    if code:
        assert lib.pkv_last_error()


def test_stream_read_validation():
    lib = ops.lib()
    assert lib.pkv_stream_read(None, 0, None, 0, None) == 0                       # nothing to read
    assert lib.pkv_stream_read(None, 16, ctypes.c_void_p(1 << 20), 4, None) == 1  # null buffer
    assert lib.pkv_stream_read(ctypes.c_void_p(1 << 20), 24, ctypes.c_void_p(1 << 20), 4, None) == 1
    assert lib.pkv_stream_read(ctypes.c_void_p((1 << 20) + 8), 32, ctypes.c_void_p(1 << 20), 4, None) == 1
    for bad in (0, 6, 262148):
        assert lib.pkv_stream_read(ctypes.c_void_p(1 << 20), 32, ctypes.c_void_p(1 << 20), bad, None) == 1


def test_sizes_beyond_the_kernels_index_range_are_refused():
    """Arguments whose products would overflow the kernels' index arithmetic
    (token rows past 2^31 - 1 bytes, tables past 2^31 - 1 tokens, pools of
    2^62 bytes or more) are refused with EUNSUPPORTED before any launch."""
    lib = ops.lib()
    huge = 1 << 50
    # decode: the table width in tokens, then the pool size
    assert _decode(lib, max_blocks=1 << 27) == 2
    assert _decode(lib, NB=huge) == 2 and b"pool" in lib.pkv_last_error()
    assert _step(lib, True, NB=huge) == 2
    # varlen: the same two limits
    p = ctypes.c_void_p(1 << 20)

    def varlen(max_blocks, nb):
        return lib.pkv_paged_attention_varlen(p, p, p, p, p, max_blocks, p, p, 2, 3, 2, 64, 8, 2, 128, nb, 16, 0.1, 1,
                                              p, 1 << 30, None)
    assert varlen(1 << 27, 16) == 2
    assert varlen(4, huge) == 2
    # cache writes: pool size and row size
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 3, 8, 128, huge, 16, 1, None) == 2
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 3, 1 << 20, 1 << 11, 16, 16, 0, None) == 2
    args = [None, 2, 4, None, None, 3, 16, None, None, None, None, 8, 128, huge, 1, None, None]
    assert lib.pkv_write_new_tokens(*args) == 2
    nul = [None] * 5
    assert lib.pkv_reshape_and_cache_fp8(*nul, 3, 1 << 20, 1 << 10, 16, 16, 0, 0.5, 0.5, None) == 2
    assert lib.pkv_reshape_and_cache_fp8(*nul, 3, 8, 128, huge, 16, 1, 0.5, 0.5, None) == 2
    # whole-block copies
    assert lib.pkv_copy_blocks(None, None, None, 2, huge, 1 << 20, None) == 2
    assert lib.pkv_swap_blocks(None, None, None, None, None, 3, 4, huge, 1 << 20, None) == 2
    # the largest legal sizes of the same calls still pass these checks (and
    # stop at the null pointers instead)
    assert lib.pkv_reshape_and_cache(None, None, None, None, None, 3, 8, 128, 1 << 30, 16, 1, None) == 1
    assert lib.pkv_copy_blocks(None, None, None, 2, 1 << 30, 1 << 20, None) == 1


def test_noalloc_decode_validation_runs_before_any_launch():
    """The allocation-free decode call rejects E4M3 pools, unsupported shapes and
    shapes whose split-K workspace exceeds its static scratch, on the host."""
    lib = ops.lib()
    assert lib.pkv_noalloc_scratch_bytes() == 16 << 20

    def call(B=2, Hq=8, Hkv=2, D=128, bs=16, dtype=1):
        p = 1 << 20
        return lib.pkv_paged_attention_decode_noalloc(p, p, p, p, p, 4, p, B, Hq, Hkv, D, 16, bs, 64, 0.1, dtype,
                                                      None)
    assert call(dtype=2) == 1
    assert call(D=96) == 2
    assert call(Hq=7) == 1
    assert call(B=9000) == 2
    assert call(B=4096, Hq=64, Hkv=8) == 2
    assert b"scratch" in lib.pkv_last_error()


def test_shared_prefix_decode_validation_runs_before_any_launch():
    lib = ops.lib()

    def call(B=2, dtype=1, groups=1 << 20, ng=1):
        p = 1 << 20
        return lib.pkv_paged_attention_decode_shared(p, p, p, p, p, 4, p, B, 8, 2, 128, 16, 16, 64, 0.1, dtype,
                                                     groups, ng, p, 1 << 30, None)
    assert call(dtype=0) == 2                          # float32 pools
    assert call(ng=2000) == 2
    assert call(ng=-1) == 1
    assert call(groups=None) == 1
    assert call(B=5000) == 2
    assert call(dtype=2) == 1                          # E4M3 needs the _fp8 call
    assert lib.pkv_decode_shared_workspace_size(2, 8, 2, 128, 16, 1, 1) > lib.pkv_decode_workspace_size(2, 8, 2, 128, 16, 1)
    assert lib.pkv_decode_shared_workspace_size(2, 8, 2, 128, 16, 0, 1) == 0
