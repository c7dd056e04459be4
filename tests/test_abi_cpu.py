"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function include/sttd.h declares, and rejects bad arguments before
touching the device."""
import ctypes
import os
import re

import pytest

from speech_text_decoder_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "sttd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sttd_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sttd.h but not exported"
    assert sorted(B.EXPORTS) == names


def test_status_strings():
    assert B.status_string(B.OK) == "ok"
    for s in range(1, 6):
        assert B.status_string(s) not in ("ok", "unknown status")
    assert B.status_string(99) == "unknown status"


def test_null_and_bad_arguments_rejected_on_host():
    L = B.lib()
    p = B.block_params(256, 4, 2, 64, 512, 1e-6, 1e6, B.BF16)
    w = B.block_weights({n: 0 for n in B.WEIGHT_SLOTS})
    assert L.sttd_block_prefill(ctypes.byref(p), ctypes.byref(w), None, None, 0, 0, 0, 1, None, 0, None) \
        == B.ERR_INVALID_ARG
    assert L.sttd_block_step(ctypes.byref(p), ctypes.byref(w), None, None, 0, 1, None, None, 1, None, None) \
        == B.ERR_INVALID_ARG
    assert L.sttd_lm_head_argmax(None, None, B.BF16, 10, 256, 1e-6, None, 1, None, 256, None, 0, None, None, None,
                                 None, None) == B.ERR_INVALID_ARG
    assert L.sttd_embed_gather(None, B.BF16, 10, 256, 1, None, None, None, None) == B.ERR_INVALID_ARG
    assert L.sttd_kv_cache_free(None) == B.ERR_INVALID_ARG
    assert L.sttd_workspace_free(None) == B.ERR_INVALID_ARG
    assert L.sttd_workspace_set_option(None, B.OPT_QKV_ATTN, 0) == B.ERR_INVALID_ARG
    out = ctypes.c_void_p()
    assert L.sttd_kv_cache_alloc(0, 1, 16, 2, 64, B.F16, ctypes.byref(out)) == B.ERR_INVALID_ARG
    assert L.sttd_kv_cache_alloc(1, 1, 16, 2, 96, B.F16, ctypes.byref(out)) == B.ERR_UNSUPPORTED
    assert L.sttd_kv_cache_alloc(1, 1, 16, 2, 64, B.BF16, ctypes.byref(out)) == B.ERR_UNSUPPORTED
    assert L.sttd_kv_cache_alloc(1 << 20, 1 << 10, 1 << 20, 8, 128, B.F16, ctypes.byref(out)) == B.ERR_OOM
    bad = B.block_params(256, 4, 3, 64, 512, 1e-6, 1e6, B.BF16)      # 4 % 3 != 0
    assert L.sttd_workspace_alloc(ctypes.byref(bad), 4, 16, 0, ctypes.byref(out)) == B.ERR_INVALID_ARG
    bad = B.block_params(256, 4, 2, 96, 512, 1e-6, 1e6, B.BF16)
    assert L.sttd_workspace_alloc(ctypes.byref(bad), 4, 16, 0, ctypes.byref(out)) == B.ERR_UNSUPPORTED
    bad = B.block_params(256, 4, 2, 64, 500, 1e-6, 1e6, B.BF16)       # ffn not a multiple of 64
    assert L.sttd_workspace_alloc(ctypes.byref(bad), 4, 16, 0, ctypes.byref(out)) == B.ERR_UNSUPPORTED
    bad = B.block_params(256, 4, 2, 64, 8256, 1e-6, 1e6, B.BF16)      # ffn above the 8192 GEMV row limit
    assert L.sttd_workspace_alloc(ctypes.byref(bad), 4, 16, 0, ctypes.byref(out)) == B.ERR_UNSUPPORTED
    bad = B.block_params(256, 72, 9, 128, 512, 1e-6, 1e6, B.BF16)     # n_heads * head_dim = 9216
    assert L.sttd_workspace_alloc(ctypes.byref(bad), 4, 16, 0, ctypes.byref(out)) == B.ERR_UNSUPPORTED


def test_kv_context_policy():
    """The cache sizing of the MOSS page's run(): 1K / 2K / 4K buckets, then
    4K steps, clamped to the ceiling (host function, no GPU)."""
    f = B.kv_context_for
    assert [f(n, 131072) for n in (1, 1024, 1025, 2048, 2049, 4096, 4097, 8192, 32769)] == \
        [1024, 1024, 2048, 2048, 4096, 4096, 8192, 8192, 36864]
    assert f(200000, 131072) == 131072 and f(3000, 2500) == 2500
    assert f(0, 1024) == 0 and f(10, 0) == 0
    # grow-only in 4K steps past 4096: never more than 4095 positions of slack
    for n in range(4097, 70000, 997):
        c = f(n, 1 << 30)
        assert c >= n and c - n < 4096 and c % 4096 == 0
