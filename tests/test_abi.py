"""C-ABI library checks that need no GPU: it loads, exports every entry point that include/dca.h
declares, and rejects bad arguments with a status code before touching the device."""
import ctypes
import os
import re

import pytest

from dual_chunk_attention_amd import dca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    """Every dca_* function declared by the headers under include/."""
    inc = os.path.join(ROOT, "include")
    names = set()
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names.update(re.findall(r"\b(dca_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_five_operations():
    names = declared_functions()
    for f in ["dca_remap_positions", "dca_rope_partial", "dca_attn_regime", "dca_lse_merge",
              "dca_attention", "dca_attention_workspace_size", "dca_attn_regime_workspace_size",
              "dca_last_error"]:
        assert f in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(dca.LIB_PATH):
        pytest.skip("libdca.so not built")
    L = dca.lib()
    for f in declared_functions():
        assert hasattr(L, f), f"{f} not exported"


def _cfg(**kw):
    base = dict(head_dim=512, n_rot=128, n_head_q=16, n_head_kv=2, chunk=1024)
    base.update(kw)
    return dca.Config(**base).c()


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=0), dca.ERR_INVALID_ARGUMENT),
    (dict(n_rot=3), dca.ERR_INVALID_ARGUMENT),
    (dict(n_rot=1024), dca.ERR_INVALID_ARGUMENT),
    (dict(n_head_q=15), dca.ERR_INVALID_ARGUMENT),
    (dict(chunk=0), dca.ERR_INVALID_ARGUMENT),
    (dict(remap_mode=3), dca.ERR_INVALID_ARGUMENT),
    (dict(remap_mode=-1), dca.ERR_INVALID_ARGUMENT),
    (dict(rope_attn_factor=0.0), dca.ERR_INVALID_ARGUMENT),
    (dict(rope_attn_factor=float("inf")), dca.ERR_INVALID_ARGUMENT),
    (dict(head_dim=256), dca.ERR_UNSUPPORTED),   # bf16 path is head_dim 512 only
    (dict(n_head_q=64, n_head_kv=1), dca.ERR_UNSUPPORTED),
])
def test_attention_rejects_bad_config(kw, code):
    if not os.path.exists(dca.LIB_PATH):
        pytest.skip("libdca.so not built")
    L = dca.lib()
    c = _cfg(**kw)
    st = L.dca_attention(ctypes.byref(c), dca.BF16, 1, 4, ctypes.c_void_p(16), ctypes.c_void_p(16),
                         ctypes.c_void_p(16), 4, dca.BF16, ctypes.c_void_p(16), None,
                         ctypes.c_void_p(16), 1 << 30, None)
    assert st == code
    assert L.dca_last_error().decode() != ""
    assert L.dca_attention_workspace_size(ctypes.byref(c), dca.BF16, 1, 4, 4) == 0


def test_other_validation_paths():
    if not os.path.exists(dca.LIB_PATH):
        pytest.skip("libdca.so not built")
    L = dca.lib()
    c = _cfg()
    vp = ctypes.c_void_p(16)
    assert L.dca_attention(ctypes.byref(c), dca.BF16, -1, 4, vp, vp, vp, 4, dca.BF16, vp, None, vp,
                           1 << 30, None) == dca.ERR_INVALID_ARGUMENT
    assert L.dca_attention(ctypes.byref(c), dca.BF16, 1, 4, None, vp, vp, 4, dca.BF16, vp, None, vp,
                           1 << 30, None) == dca.ERR_INVALID_ARGUMENT
    need = L.dca_attention_workspace_size(ctypes.byref(c), dca.BF16, 1, 4096, 4096)
    assert need > 0
    assert L.dca_attention(ctypes.byref(c), dca.BF16, 1, 4096, vp, vp, vp, 4096, dca.BF16, vp, None,
                           vp, need - 1, None) == dca.ERR_WORKSPACE_TOO_SMALL
    assert L.dca_attn_regime(ctypes.byref(c), dca.BF16, 3, 1, 4, vp, vp, vp, vp, 4, vp, vp, None, 0,
                             None) == dca.ERR_INVALID_ARGUMENT
    parts = (ctypes.c_void_p * 9)(*([16] * 9))
    assert L.dca_lse_merge(9, parts, parts, 4, 512, dca.F32, vp, vp, None) == dca.ERR_INVALID_ARGUMENT
    assert L.dca_lse_merge(0, parts, parts, 4, 512, dca.F32, vp, vp, None) == dca.ERR_INVALID_ARGUMENT
    c0 = _cfg(chunk=0)
    assert L.dca_remap_positions(ctypes.byref(c0), 1, 4, vp, 4, vp, vp, vp, None) == dca.ERR_INVALID_ARGUMENT
    assert L.dca_rope_partial(ctypes.byref(c), 7, vp, 4, 2, vp, vp, None) == dca.ERR_INVALID_ARGUMENT
    # empty work is a no-op that succeeds
    assert L.dca_attention(ctypes.byref(c), dca.BF16, 0, 4, None, None, None, 4, dca.BF16, None,
                           None, None, 0, None) == dca.OK


def test_q8_entry_point_validation():
    if not os.path.exists(dca.LIB_PATH):
        pytest.skip("libdca.so not built")
    L = dca.lib()
    c = _cfg()
    vp = ctypes.c_void_p(16)
    need = L.dca_attention_q8_workspace_size(ctypes.byref(c), 8, 1, 262144)
    # split-KV partials for every T: 3 regimes x 64 spans of 4096 keys x 128 (row, head) x 512 fp32
    assert need >= 3 * 64 * 128 * 512 * 4
    assert L.dca_attention_q8(ctypes.byref(c), 8, 1, vp, vp, vp, vp, 262144, dca.BF16, vp, None, vp,
                              need - 1, None) == dca.ERR_WORKSPACE_TOO_SMALL
    assert L.dca_attention_q8(ctypes.byref(c), 8, 1, vp, vp, vp, None, 262144, dca.BF16, vp, None, vp,
                              need, None) == dca.ERR_INVALID_ARGUMENT     # scales missing
    assert L.dca_attention_q8(ctypes.byref(c), 8, 1, vp, vp, vp, vp, 262144, 7, vp, None, vp,
                              need, None) == dca.ERR_INVALID_ARGUMENT     # bad output dtype
    bad = _cfg(head_dim=256)
    assert L.dca_attention_q8(ctypes.byref(bad), 8, 1, vp, vp, vp, vp, 4, dca.BF16, vp, None, vp,
                              1 << 30, None) == dca.ERR_UNSUPPORTED
    assert L.dca_attention_q8_workspace_size(ctypes.byref(bad), 8, 1, 4) == 0
    # more (row, KV head) pairs than the split-KV grid takes
    assert L.dca_attention_q8(ctypes.byref(c), 40000, 1, vp, vp, vp, vp, 4, dca.BF16, vp, None, vp,
                              1 << 40, None) == dca.ERR_UNSUPPORTED
    assert L.dca_attention_q8(ctypes.byref(c), 0, 1, None, None, None, None, 4, dca.BF16, None, None,
                              None, 0, None) == dca.OK


def test_q4_entry_point_validation():
    if not os.path.exists(dca.LIB_PATH):
        pytest.skip("libdca.so not built")
    L = dca.lib()
    c = _cfg()
    vp = ctypes.c_void_p(16)
    need = L.dca_attention_q4_workspace_size(ctypes.byref(c), 8, 1, 262144)
    assert need == L.dca_attention_q8_workspace_size(ctypes.byref(c), 8, 1, 262144) > 0
    assert L.dca_attention_q4(ctypes.byref(c), 8, 1, vp, vp, vp, vp, 262144, dca.BF16, vp, None, vp,
                              need - 1, None) == dca.ERR_WORKSPACE_TOO_SMALL
    assert L.dca_attention_q4(ctypes.byref(c), 8, 1, vp, vp, None, vp, 262144, dca.BF16, vp, None, vp,
                              need, None) == dca.ERR_INVALID_ARGUMENT     # codes missing
    assert L.dca_attention_q4(ctypes.byref(c), 0, 1, None, None, None, None, 4, dca.BF16, None, None,
                              None, 0, None) == dca.OK


def test_window_entry_point_validation():
    """Host-side checks of dca_attention_window that return before any runtime call."""
    if not os.path.exists(dca.LIB_PATH):
        pytest.skip("libdca.so not built")
    L = dca.lib()
    c = _cfg(chunk=65536)
    vp = ctypes.c_void_p(16)
    win = dca._Region(dca.KV_BF16, 16, None, 65536)
    tail = dca._Region(dca.KV_Q4_0, 16, 16, 196608)
    need = L.dca_attention_window_workspace_size(ctypes.byref(c), 8, 1, 65536, 196608)
    # span 4096: 16 window spans + 48 tail spans, 3 regimes of fp32 partials [8*16, 512]
    assert need >= 3 * 64 * 128 * 512 * 4
    args = lambda w, t, ws: (ctypes.byref(c), 8, 1, vp, vp, ctypes.byref(w), ctypes.byref(t), dca.BF16,
                             vp, None, vp, ws, None)
    assert L.dca_attention_window(*args(win, tail, need - 1)) == dca.ERR_WORKSPACE_TOO_SMALL
    assert L.dca_attention_window(*args(win, dca._Region(dca.KV_Q4_0, 16, None, 10), need)) \
        == dca.ERR_INVALID_ARGUMENT                                       # q4_0 region without scales
    assert L.dca_attention_window(*args(win, dca._Region(7, 16, 16, 10), need)) == dca.ERR_INVALID_ARGUMENT
    assert L.dca_attention_window(*args(win, dca._Region(dca.KV_BF16, 16, None, -1), need)) \
        == dca.ERR_INVALID_ARGUMENT
    assert L.dca_attention_window(ctypes.byref(c), 8, 1, vp, vp, None, ctypes.byref(tail), dca.BF16, vp,
                                  None, vp, need, None) == dca.ERR_INVALID_ARGUMENT
    empty = dca._Region(dca.KV_BF16, None, None, 0)
    assert L.dca_attention_window(ctypes.byref(c), 0, 1, None, None, ctypes.byref(empty),
                                  ctypes.byref(empty), dca.BF16, None, None, None, 0, None) == dca.OK


def test_unaligned_pointers_rejected_before_any_launch():
    """The bf16 and quantized paths stream rows with 16-byte accesses: a pointer off a 16-byte
    boundary (q, k, codes, scales, o, workspace, region keys) is an invalid argument, caught on the
    host; the fp32 path takes it."""
    if not os.path.exists(dca.LIB_PATH):
        pytest.skip("libdca.so not built")
    L = dca.lib()
    c = _cfg()
    ok, odd = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8)
    need = L.dca_attention_workspace_size(ctypes.byref(c), dca.BF16, 1, 64, 64)
    for i in range(4):   # q, k, o, workspace in turn
        p = [ok] * 4
        p[i] = odd
        assert L.dca_attention(ctypes.byref(c), dca.BF16, 1, 64, p[0], ok, p[1], 64, dca.BF16, p[2],
                               None, p[3], need, None) == dca.ERR_INVALID_ARGUMENT
        assert "16-byte aligned" in L.dca_last_error().decode()
    need_r = max(L.dca_attn_regime_workspace_size(ctypes.byref(c), dca.BF16, 1, 64, 64), 1)
    assert L.dca_attn_regime(ctypes.byref(c), dca.BF16, 0, 1, 64, odd, ok, ok, ok, 64, ok, ok, ok,
                             need_r, None) == dca.ERR_INVALID_ARGUMENT
    need8 = L.dca_attention_q8_workspace_size(ctypes.byref(c), 1, 1, 64)
    for i in range(5):   # q, codes, scales, o, workspace
        p = [ok] * 5
        p[i] = odd
        assert L.dca_attention_q8(ctypes.byref(c), 1, 1, p[0], ok, p[1], p[2], 64, dca.BF16, p[3], None,
                                  p[4], need8, None) == dca.ERR_INVALID_ARGUMENT
        assert L.dca_attention_q4(ctypes.byref(c), 1, 1, p[0], ok, p[1], p[2], 64, dca.BF16, p[3], None,
                                  p[4], need8, None) == dca.ERR_INVALID_ARGUMENT
    needw = L.dca_attention_window_workspace_size(ctypes.byref(c), 1, 1, 32, 32)
    good = dca._Region(dca.KV_BF16, 4096, None, 32)
    bad = dca._Region(dca.KV_Q8_0, 4096, 4096 + 8, 32)
    assert L.dca_attention_window(ctypes.byref(c), 1, 1, ok, ok, ctypes.byref(good), ctypes.byref(bad),
                                  dca.BF16, ok, None, ok, needw, None) == dca.ERR_INVALID_ARGUMENT
