"""The C-ABI library loads without a GPU, exports every entry point that
include/flashloop.h declares, and rejects invalid arguments on the host
before enqueuing anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from sparse_attention_kv_amd import fl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashloop.h")

FAKE = 0x10000  # a non-null pointer value; never dereferenced by host validation


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fl_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fl.LIB_PATH):
        from sparse_attention_kv_amd import build
        build.build()
    return fl.lib()


def test_exports_match_header(L):
    declared = _declared()
    assert set(fl.EXPORTS) == set(declared), declared
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_workspace(L):
    assert "gfx950" in fl.fl_version()
    assert fl.fl_workspace_size(fl.FL_WS_SPARSE_ATTN, 16, 2048, 128, 4) >= 4 * 16 * 2048 * 128 * 2
    assert fl.fl_workspace_size(fl.FL_WS_SPARSE_ATTN, 16, 2048, 96, 4) == 0
    assert fl.fl_workspace_size(99, 1, 1, 1, 1) == 0


def _err(L):
    return L.fl_last_error().decode()


def test_select_active_rejects(L):
    rc = L.fl_select_active(1, 0, FAKE, FAKE, 100, 64, None, 100, 0, None, FAKE, FAKE, None, None, 0, None)
    assert rc == -1 and "n_select" in _err(L)
    rc = L.fl_select_active(1, 0, FAKE, FAKE, 100, 64, None, 101, 5, None, FAKE, FAKE, None, None, 0, None)
    assert rc == -1 and "n_cand" in _err(L)
    rc = L.fl_select_active(1, 0, FAKE, FAKE, 100, 60, None, 100, 5, None, FAKE, FAKE, None, None, 0, None)
    assert rc == -1 and "multiple of 8" in _err(L)
    rc = L.fl_select_active(1, 0, None, FAKE, 100, 64, None, 100, 5, None, FAKE, FAKE, None, None, 0, None)
    assert rc == -1
    rc = L.fl_select_active(1, 2, FAKE, FAKE, 100, 64, None, 100, 5, None, FAKE, FAKE, None, None, 0, None)
    assert rc == -1 and "stat_kind" in _err(L)


def test_select_columns_rejects(L):
    assert L.fl_select_columns(FAKE, None, 2, 100, 4, 4, FAKE, None, 0, None) == -1
    assert L.fl_select_columns(FAKE, None, 2, 100, -1, 10, FAKE, None, 0, None) == -1
    assert L.fl_select_columns(None, None, 2, 100, 4, 10, FAKE, None, 0, None) == -1
    assert L.fl_select_columns(FAKE, None, 0, 100, 4, 10, FAKE, None, 0, None) == -1


def _cache(N=64, H=2, d=128, g=64, bits=(8, 4)):
    c = fl.FlKvCache()
    c.N, c.H, c.d, c.g, c.n_levels = N, H, d, g, len(bits)
    for l, b in enumerate(bits):
        L = c.level[l]
        L.bits, L.n_rows = b, N if l == 0 else N // 2
        L.rows = None if l == 0 else FAKE
        L.slot = None if l == 0 else FAKE
        L.k_codes = L.v_codes = L.k_scale = L.v_scale = FAKE
    return c


def test_quant_rejects(L):
    c = _cache(d=96)
    assert L.fl_kv_residual_quant(ctypes.byref(c), 0, 1, FAKE, FAKE, 0, None) == -2
    c = _cache(bits=(8, 3))
    assert L.fl_kv_residual_quant(ctypes.byref(c), 1, 1, FAKE, FAKE, 0, None) == -2
    c = _cache(bits=(4,))
    assert L.fl_kv_residual_quant(ctypes.byref(c), 0, 1, FAKE, FAKE, 0, None) == -2
    c = _cache()
    c.level[1].slot = None
    assert L.fl_kv_residual_quant(ctypes.byref(c), 1, 1, FAKE, FAKE, 0, None) == -1
    c = _cache(g=48)
    assert L.fl_kv_residual_quant(ctypes.byref(c), 0, 1, FAKE, FAKE, 0, None) == -2
    assert L.fl_kv_residual_quant(None, 0, 1, FAKE, FAKE, 0, None) == -1
    c = _cache()
    assert L.fl_kv_residual_quant(ctypes.byref(c), 0, 7, FAKE, FAKE, 0, None) == -1   # dtype


def _args(**kw):
    a = fl.FlAttnArgs()
    a.dtype, a.q, a.active, a.n, a.sel, a.k = 1, FAKE, FAKE, 10, FAKE, 8
    a.sm, a.level, a.mode, a.cache_op = 0.125, 1, 0, 0
    a.out = a.lse = a.mass_u = a.out_u = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_attn_rejects(L):
    c = _cache()
    a = _args()
    ws = ctypes.create_string_buffer(64)
    assert L.fl_sparse_loop_attn(ctypes.byref(c), ctypes.byref(a), ctypes.addressof(ws), 64, None) == -3
    assert "workspace" in _err(L)
    a = _args(sel=None)
    assert L.fl_sparse_loop_attn(ctypes.byref(c), ctypes.byref(a), None, 0, None) == -1
    a = _args(cache_op=2, q_prev=None)
    assert L.fl_sparse_loop_attn(ctypes.byref(c), ctypes.byref(a), None, 0, None) == -1
    a = _args(cache_op=2, level=0, q_prev=FAKE)
    assert L.fl_sparse_loop_attn(ctypes.byref(c), ctypes.byref(a), None, 0, None) == -1
    a = _args(mode=2)
    assert L.fl_sparse_loop_attn(ctypes.byref(c), ctypes.byref(a), None, 0, None) in (-2, -3)
    a = _args(n=0)
    assert L.fl_sparse_loop_attn(ctypes.byref(c), ctypes.byref(a), None, 0, None) == -1
    a = _args(col_stat_kind=2)
    assert L.fl_sparse_loop_attn(ctypes.byref(c), ctypes.byref(a), None, 0, None) == -1
    assert "col_stat_kind" in _err(L)


def test_block_step_rejects(L):
    cfg = fl.FlBlockCfg()
    cfg.N, cfg.H, cfg.d, cfg.g, cfg.R, cfg.n_layers, cfg.ffn = 64, 2, 128, 64, 2, 1, 512
    st = fl.FlBlockState()
    W = (fl.FlLayerWeights * 1)()
    layers = (fl.FlLayerState * 1)()
    st.layers = ctypes.cast(layers, ctypes.POINTER(fl.FlLayerState))
    assert L.fl_block_step(ctypes.byref(cfg), W, ctypes.byref(st), 3, None, 0, None) == -1
    assert L.fl_block_step(ctypes.byref(cfg), W, ctypes.byref(st), 1, None, 0, None) == -1  # h NULL
    st.h = st.h_entry = st.stat = FAKE
    assert L.fl_block_step(ctypes.byref(cfg), W, ctypes.byref(st), 1, None, 0, None) == -3  # workspace
    cfg.ffn = 500
    assert L.fl_block_step(ctypes.byref(cfg), W, ctypes.byref(st), 1, None, 0, None) == -2
    cfg.ffn, cfg.d = 512, 96
    assert L.fl_block_step(ctypes.byref(cfg), W, ctypes.byref(st), 1, None, 0, None) == -2
    cfg.d, cfg.token_stat = 128, 2
    assert L.fl_block_step(ctypes.byref(cfg), W, ctypes.byref(st), 1, None, 0, None) == -1
    assert "token_stat" in _err(L)
    cfg.token_stat = 0
    assert fl.fl_workspace_size(fl.FL_WS_BLOCK_STEP, 8192, 16, 128, 5632) > 8192 * 2048 * 2 * 5


def test_loop_step_rejects(L):
    cfg = fl.FlLoopCfg()
    cfg.N, cfg.H, cfg.d, cfg.g, cfg.R = 64, 2, 128, 64, 2
    st = fl.FlLoopState()
    inp = fl.FlLoopInputs()
    assert L.fl_loop_step(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(inp), 3, None, 0, None) == -1
    assert L.fl_loop_step(None, ctypes.byref(st), ctypes.byref(inp), 1, None, 0, None) == -1
    cfg.col_stat = 7
    assert L.fl_loop_step(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(inp), 1, None, 0, None) == -1
    assert "col_stat" in _err(L)
    cfg.col_stat = 0
    st.cache.N, st.cache.H, st.cache.d, st.cache.g = 64, 2, 128, 64
    assert L.fl_loop_step(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(inp), 1, None, 0, None) == -1
    assert "q/k/v" in _err(L)


def test_decode_step_rejects(L):
    cfg = fl.FlDecodeCfg()
    cfg.B, cfg.N, cfg.H, cfg.d, cfg.g, cfg.R, cfg.n_sink = 2, 64, 2, 128, 64, 2, 4
    st = fl.FlDecodeState()
    inp = fl.FlDecodeInputs()
    assert L.fl_decode_step(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(inp), 3, None) == -1
    assert L.fl_decode_step(None, ctypes.byref(st), ctypes.byref(inp), 1, None) == -1
    assert L.fl_decode_step(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(inp), 1, None) == -1
    assert "cache dims" in _err(L)
    cfg.N = 20000
    assert L.fl_decode_step(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(inp), 1, None) == -1
    assert "LDS" in _err(L)
    cfg.N = 64
    st.cache = _cache(N=64, H=2, d=128, g=64, bits=(8, 4))
    assert L.fl_decode_step(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(inp), 1, None) == -1
    assert "q/k_self/v_self" in _err(L)


def test_decode_append_rejects(L):
    cfg = fl.FlDecodeCfg()
    cfg.B, cfg.N, cfg.H, cfg.d, cfg.g, cfg.R, cfg.n_sink = 2, 64, 2, 128, 64, 2, 4
    cfg.N_cap, cfg.rows_cap[1] = 256, 200
    st = fl.FlDecodeState()
    st.cache = _cache(N=64, bits=(4, 4))
    st.cache.scheme = fl.FL_QUANT_ASYM
    for lv in range(2):
        st.cache.level[lv].k_zero = st.cache.level[lv].v_zero = FAKE
    win = fl.FlDecodeWindow()
    win.cap, win.count = 128, 128
    for lv in range(2):
        win.k[lv] = win.v[lv] = FAKE
    app = lambda slot, n: L.fl_decode_append(ctypes.byref(cfg), ctypes.byref(st), ctypes.byref(win),
                                             slot, n, None)
    # one token cannot complete a per-channel key group of g rows
    assert app(0, 1) == -2 and "key group" in _err(L)
    # level 1 holds 32 rows: with the default origin 0 a block would straddle
    # the prompt's partial group
    assert app(0, 64) == -1 and "does not start a key group" in _err(L)
    cfg.key_group_origin[1] = 300
    assert app(0, 64) == -1 and "key_group_origin" in _err(L)
    cfg.key_group_origin[1] = 32
    assert app(128, 64) == -1 and "slot" in _err(L)
    cfg.N_cap = 100
    assert app(0, 64) == -1 and "N_cap" in _err(L)
    # absmax: the base must be int8
    st.cache.scheme = fl.FL_QUANT_ABSMAX
    assert app(0, 1) == -2 and "base level bits 4" in _err(L)


def test_check_indices_host(L):
    import numpy as np
    ok = np.array([0, 3, 4, 9], np.int32)
    assert fl.fl_check_indices(ok, 0, 10) == (0, "")
    assert fl.fl_check_indices(np.zeros(0, np.int32), 0, 10)[0] == 0
    rc, msg = fl.fl_check_indices(np.array([0, 4, 3], np.int32), 0, 10)
    assert rc == -1 and "element 2 = 3" in msg and "ascending" in msg
    rc, msg = fl.fl_check_indices(np.array([1, 1], np.int32), 0, 10)
    assert rc == -1 and "element 1 = 1" in msg                    # duplicate
    rc, msg = fl.fl_check_indices(np.array([2, 10], np.int32), 0, 10)
    assert rc == -1 and "outside [0, 10)" in msg
    rc, msg = fl.fl_check_indices(np.array([-1, 2], np.int32), 0, 10)
    assert rc == -1 and "element 0 = -1" in msg


def test_check_finite_host(L):
    import numpy as np
    assert fl.fl_check_finite(np.array([0.0, -1.5, 3e38], np.float32)) == (0, "")
    for bad in (np.nan, np.inf, -np.inf):
        rc, msg = fl.fl_check_finite(np.array([1.0, bad], np.float32))
        assert rc == -1 and "element 1" in msg and "finite" in msg
    assert L.fl_check_finite(None, 3) == -1
    assert L.fl_check_indices(None, 3, 0, 1) == -1


def test_check_mode_toggles(L):
    fl.fl_set_checks(True)
    try:
        # host-side argument validation still comes first (nothing is copied)
        rc = L.fl_select_active(1, 0, FAKE, FAKE, 100, 64, None, 100, 0, None, FAKE, FAKE, None,
                                None, 0, None)
        assert rc == -1 and "n_select" in _err(L)
    finally:
        fl.fl_set_checks(False)
