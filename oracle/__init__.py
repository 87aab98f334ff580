"""FlashLoop oracle: plain fp32 CPU reference of the lazy-update loop step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library ``sparse_attention_kv_amd`` and never imports it.

The arithmetic lives in ``flo_oracle.c`` (plain C, fp32, program-order
evaluation); this module loads it with ctypes and chains the per-step
functions into whole loops (``loop.py``).  Section references are to the
FlashLoop paper (arXiv 2609.29812): Sec. 4.1 token-sparse updates, Sec. 4.2
loop-aware sparse attention, Sec. 4.3 / App. E KV residual quantisation.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (brute-force selection, quantiser bounds and a
hand-worked golden group, reduction to textbook dense attention through an
independent library routine, unchanged-input / conservation / column-total
invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flo_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no intrinsics, no fast-math, no FMA)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p
_int = ctypes.c_int
_long = ctypes.c_long
_flt = ctypes.c_float


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.flo_num_threads.restype = _int
        L.flo_active_count.argtypes = [ctypes.c_double, _int, _int]
        L.flo_active_count.restype = _int
        L.flo_delta_norm.argtypes = [_f32p, _f32p, _int, _vp, _int, _f32p]
        L.flo_delta_norm_rel.argtypes = [_f32p, _f32p, _int, _vp, _int, _f32p]
        L.flo_top_select.argtypes = [_f32p, _vp, _int, _int, _i32p]
        L.flo_top_select.restype = _int
        L.flo_select_columns.argtypes = [_f32p, _vp, _int, _int, _int, _int, _i32p]
        L.flo_select_columns.restype = _int
        L.flo_quant_group.argtypes = [_f32p, _int, _int, _i8p, _f32p]
        L.flo_quantize_rows.argtypes = [_f32p, _vp, _long, _int, _int, _int, _int,
                                        _vp, _vp, _vp, _f32p]
        L.flo_pack_codes.argtypes = [_i8p, _long, _int, _u8p]
        L.flo_quant_asym_group.argtypes = [_f32p, _int, _long, _int, _u8p, _long, _f32p, _f32p]
        L.flo_quantize_rows_asym.argtypes = [_f32p, _vp, _long, _int, _int, _int, _int, _int,
                                             _u8p, _f32p, _f32p, _f32p]
        L.flo_attend.argtypes = [_int, _int, _int, _flt, _f32p, _f32p, _f32p, _vp, _int,
                                 _vp, _int, _vp, _vp, _f32p, _f32p]
        L.flo_unselected_cache.argtypes = [_int, _int, _int, _flt, _f32p, _f32p, _f32p,
                                           _i32p, _int, _vp, _int, _i32p, _int, _f32p,
                                           _vp, _vp, _f32p, _f32p]
        L.flo_column_stats.argtypes = [_int, _int, _int, _flt, _f32p, _f32p, _vp, _int,
                                       _vp, _int, _f32p, _vp, _vp, _f32p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def num_threads() -> int:
    return lib().flo_num_threads()


def active_count(rho: float, N: int, n_prev: int) -> int:
    """Sec. 4.1: number of active tokens kept in a loop (ceil(rho*N), nested)."""
    return lib().flo_active_count(float(rho), int(N), int(n_prev))


def delta_norm(h_cur, h_prev, cand=None, relative=False):
    """Sec. 4.1: ||h_r(i) - h_{r-1}(i)||_2 over candidate rows (fp32); with
    relative=True the normalised change ||h_r(i) - h_{r-1}(i)|| / ||h_{r-1}(i)||
    (0 for an unchanged zero state, +inf for a changed one)."""
    h_cur = _c(h_cur, np.float32)
    h_prev = _c(h_prev, np.float32)
    N, D = h_cur.shape
    cand_a = None if cand is None else _c(cand, np.int32)
    n = N if cand is None else len(cand_a)
    out = np.empty(n, np.float32)
    fn = lib().flo_delta_norm_rel if relative else lib().flo_delta_norm
    fn(h_cur, h_prev, D, _ptr(cand_a), n, out)
    return out


def top_select(key, n_sel, pos=None):
    """Top n_sel by (key desc, position asc), returned in ascending position."""
    key = _c(key, np.float32)
    pos_a = None if pos is None else _c(pos, np.int32)
    out = np.empty(n_sel, np.int32)
    if lib().flo_top_select(key, _ptr(pos_a), len(key), int(n_sel), out) != 0:
        raise ValueError("top_select: NaN key or n_sel out of range")
    return out


def select_columns(cstat, sel_prev, k, n_sink):
    """Sec. 4.2: nested column selection with n_sink always-kept sinks.

    cstat: [H][k_prev] aligned with sel_prev ([H][k_prev] or None = all)."""
    cstat = _c(cstat, np.float32)
    H, k_prev = cstat.shape
    sp = None if sel_prev is None else _c(sel_prev, np.int32)
    k_out = min(k, k_prev)
    out = np.empty((H, k_out), np.int32)
    if lib().flo_select_columns(cstat, _ptr(sp), H, k_prev, int(n_sink), int(k), out) != 0:
        raise ValueError("select_columns: bad input")
    return out


def quant_group(x, bits):
    x = _c(x, np.float32)
    code = np.empty(len(x), np.int8)
    s = np.empty(1, np.float32)
    lib().flo_quant_group(x, len(x), int(bits), code, s)
    return code, s[0]


def quantize_rows(x_new, xhat_prev, g, bits):
    """Sec. 3.3/4.3: one base (xhat_prev None) or residual level for [n][H][d] rows.

    Returns (codes int8 [n][H][d] or None, scales [n][H][d/g] or None,
    raw fp32 residual [n][H][d] or None, xhat [n][H][d])."""
    x_new = _c(x_new, np.float32)
    n, H, d = x_new.shape
    xp = None if xhat_prev is None else _c(xhat_prev, np.float32)
    xhat = np.empty_like(x_new)
    if bits == 32:
        raw = np.empty_like(x_new)
        lib().flo_quantize_rows(x_new, _ptr(xp), n, H, d, g, 32, None, None, _ptr(raw), xhat)
        return None, None, raw, xhat
    codes = np.empty((n, H, d), np.int8)
    scales = np.empty((n, H, d // g), np.float32)
    lib().flo_quantize_rows(x_new, _ptr(xp), n, H, d, g, int(bits), _ptr(codes),
                            _ptr(scales), None, xhat)
    return codes, scales, None, xhat


def quant_asym_group(x, bits):
    """App. E: one asymmetric min/max group -> (unsigned codes, scale, zero)."""
    x = _c(x, np.float32)
    code = np.empty(len(x), np.uint8)
    s = np.empty(1, np.float32); z = np.empty(1, np.float32)
    lib().flo_quant_asym_group(x, len(x), 1, int(bits), code, 1, s, z)
    return code, s[0], z[0]


def quantize_rows_asym(x_new, xhat_prev, g, bits, per_channel):
    """App. E: one level under the paper's quantiser for [n][H][d] packed rows.

    per_channel=True (keys): groups of g consecutive rows per (head, channel),
    scales/zeros [ceil(n/g)][H][d]; False (values): groups of g channels per
    (row, head), scales/zeros [n][H][d/g].  Returns (codes uint8 [n][H][d],
    scales, zeros, xhat)."""
    x_new = _c(x_new, np.float32)
    n, H, d = x_new.shape
    xp = None if xhat_prev is None else _c(xhat_prev, np.float32)
    shp = ((n + g - 1) // g, H, d) if per_channel else (n, H, d // g)
    codes = np.empty((n, H, d), np.uint8)
    scales = np.empty(shp, np.float32)
    zeros = np.empty(shp, np.float32)
    xhat = np.empty_like(x_new)
    lib().flo_quantize_rows_asym(x_new, _ptr(xp), n, H, d, g, int(bits), int(bool(per_channel)),
                                 codes, scales, zeros, xhat)
    return codes, scales, zeros, xhat


def pack_codes(codes, bits):
    codes = np.asarray(codes)
    if codes.dtype == np.uint8:          # unsigned codes: same bits
        codes = codes.view(np.int8)
    codes = _c(codes, np.int8)
    flat = codes.reshape(-1)
    out = np.empty(len(flat) * bits // 8, np.uint8)
    lib().flo_pack_codes(flat, len(flat), int(bits), out)
    return out.reshape(*codes.shape[:-1], codes.shape[-1] * bits // 8)


def attend(q, khat, vhat, rows, sel, sm, mass_u=None, out_u=None):
    """Sec. 4.2: sparse (sel given) or dense (sel None) causal attention.

    q/khat/vhat [N][H][d] by position; rows [n] ascending (None = all);
    returns out [n][H][d], lse [n][H]."""
    q = _c(q, np.float32); khat = _c(khat, np.float32); vhat = _c(vhat, np.float32)
    N, H, d = q.shape
    rows_a = None if rows is None else _c(rows, np.int32)
    n = N if rows is None else len(rows_a)
    sel_a = None if sel is None else _c(sel, np.int32)
    k = N if sel is None else sel_a.shape[1]
    mu = None if mass_u is None else _c(mass_u, np.float32)
    ou = None if out_u is None else _c(out_u, np.float32)
    out = np.empty((n, H, d), np.float32)
    lse = np.empty((n, H), np.float32)
    lib().flo_attend(N, H, d, float(sm), q, khat, vhat, _ptr(rows_a), n, _ptr(sel_a), k,
                     _ptr(mu), _ptr(ou), out, lse)
    return out, lse


def unselected_cache(q_prev, khat_prev, vhat_prev, rows, sel_prev, sel_new, lse_prev,
                     sm, mass_u_prev=None, out_u_prev=None):
    """Sec. 4.2: mass and partial output of the columns pruned at this loop
    (additive form) under the previous loop's distribution."""
    q_prev = _c(q_prev, np.float32); khat_prev = _c(khat_prev, np.float32)
    vhat_prev = _c(vhat_prev, np.float32)
    N, H, d = q_prev.shape
    rows_a = _c(rows, np.int32)
    n = len(rows_a)
    sp = None if sel_prev is None else _c(sel_prev, np.int32)
    k_prev = N if sel_prev is None else sp.shape[1]
    sn = _c(sel_new, np.int32)
    mu_p = None if mass_u_prev is None else _c(mass_u_prev, np.float32)
    ou_p = None if out_u_prev is None else _c(out_u_prev, np.float32)
    mass_u = np.empty((n, H), np.float32)
    out_u = np.empty((n, H, d), np.float32)
    lib().flo_unselected_cache(N, H, d, float(sm), q_prev, khat_prev, vhat_prev, rows_a, n,
                               _ptr(sp), k_prev, sn, sn.shape[1], _c(lse_prev, np.float32),
                               _ptr(mu_p), _ptr(ou_p), mass_u, out_u)
    return mass_u, out_u


def column_stats(q, khat, rows, sel, lse, sm, mass_u=None, vhat=None):
    """Sec. 4.2: per-head column mass summed over this loop's rows -> [H][k];
    with vhat ([N][H][d]) each column's mass is weighted by ||vhat(j)||."""
    q = _c(q, np.float32); khat = _c(khat, np.float32)
    N, H, d = q.shape
    rows_a = None if rows is None else _c(rows, np.int32)
    n = N if rows is None else len(rows_a)
    sel_a = None if sel is None else _c(sel, np.int32)
    k = N if sel is None else sel_a.shape[1]
    mu = None if mass_u is None else _c(mass_u, np.float32)
    vh = None if vhat is None else _c(vhat, np.float32)
    out = np.empty((H, k), np.float32)
    lib().flo_column_stats(N, H, d, float(sm), q, khat, _ptr(rows_a), n, _ptr(sel_a), k,
                           _c(lse, np.float32), _ptr(mu), _ptr(vh), out)
    return out
