"""ctypes binding of libflashloop.so (C ABI in include/flashloop.h).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  PyTorch provides device memory (tensors' data pointers) and the
stream (torch's current HIP stream).  The library must be built
(``python -m sparse_attention_kv_amd.build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_long, c_size_t, c_void_p

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflashloop.so")

FL_F32, FL_BF16 = 0, 1
FL_DEQ_AUTO, FL_DEQ_ONCE, FL_DEQ_IN_TILE = 0, 1, 2
FL_CACHE_CARRY, FL_CACHE_ZERO, FL_CACHE_REBUILD = 0, 1, 2
FL_TOKEN_STAT_ABS, FL_TOKEN_STAT_REL = 0, 1
FL_COL_STAT_MASS, FL_COL_STAT_VNORM = 0, 1
FL_QUANT_ABSMAX, FL_QUANT_ASYM = 0, 1
FL_WS_SELECT_ACTIVE, FL_WS_SELECT_COLUMNS, FL_WS_SPARSE_ATTN, FL_WS_LOOP_STEP = 1, 2, 3, 4
MAX_LEVELS = 32

EXPORTS = ["fl_select_active", "fl_select_columns", "fl_kv_residual_quant",
           "fl_sparse_loop_attn", "fl_loop_step", "fl_block_step", "fl_decode_step",
           "fl_decode_append", "fl_sq_err", "fl_kv_dequant", "fl_workspace_size",
           "fl_last_error", "fl_version", "fl_timing_enable", "fl_timing_report",
           "fl_check_indices", "fl_check_finite", "fl_set_checks", "fl_sparse_loop_attn_noalloc"]
FL_WS_BLOCK_STEP = 5
FL_WS_SQ_ERR = 6


class FlError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} -> {code}: {msg}")
        self.code = code


class FlKvLevel(ctypes.Structure):
    _fields_ = [("bits", c_int), ("n_rows", c_int), ("rows", c_void_p), ("slot", c_void_p),
                ("k_codes", c_void_p), ("v_codes", c_void_p), ("k_scale", c_void_p),
                ("v_scale", c_void_p), ("k_zero", c_void_p), ("v_zero", c_void_p)]


class FlKvCache(ctypes.Structure):
    _fields_ = [("N", c_int), ("H", c_int), ("d", c_int), ("g", c_int), ("n_levels", c_int),
                ("scheme", c_int), ("level", FlKvLevel * MAX_LEVELS), ("cls", c_void_p)]


class FlAttnArgs(ctypes.Structure):
    _fields_ = [("dtype", c_int), ("q", c_void_p), ("q_gathered", c_int), ("active", c_void_p),
                ("n", c_int), ("sel", c_void_p), ("k", c_int), ("sm", c_float),
                ("level", c_int), ("mode", c_int), ("cache_op", c_int), ("out", c_void_p),
                ("lse", c_void_p), ("mass_u", c_void_p), ("out_u", c_void_p),
                ("col_stat", c_void_p), ("q_prev", c_void_p), ("q_prev_gathered", c_int),
                ("col_stat_kind", c_int), ("sel_prev", c_void_p), ("k_prev", c_int),
                ("cls_current", c_int)]


class FlLoopCfg(ctypes.Structure):
    _fields_ = [("N", c_int), ("H", c_int), ("d", c_int), ("g", c_int), ("R", c_int),
                ("n_sink", c_int), ("dtype", c_int), ("n_active", c_int * MAX_LEVELS),
                ("k_cols", c_int * MAX_LEVELS), ("bits", c_int * MAX_LEVELS), ("mode", c_int),
                ("token_stat", c_int), ("col_stat", c_int)]


class FlLoopState(ctypes.Structure):
    _fields_ = [("cache", FlKvCache), ("active", c_void_p * MAX_LEVELS),
                ("slot", c_void_p * MAX_LEVELS), ("stat", c_void_p),
                ("sel", c_void_p * MAX_LEVELS), ("sel_used", c_void_p * MAX_LEVELS),
                ("k_cur", c_int * MAX_LEVELS), ("col_stat", c_void_p * MAX_LEVELS),
                ("out", c_void_p), ("lse", c_void_p), ("mass_u", c_void_p), ("out_u", c_void_p)]


class FlLoopInputs(ctypes.Structure):
    _fields_ = [("h_cur", c_void_p), ("h_prev", c_void_p), ("q", c_void_p), ("k", c_void_p),
                ("v", c_void_p), ("q_prev", c_void_p)]


class FlBlockCfg(ctypes.Structure):
    _fields_ = [("N", c_int), ("H", c_int), ("d", c_int), ("g", c_int), ("R", c_int),
                ("n_sink", c_int), ("n_layers", c_int), ("ffn", c_int), ("rope_theta", c_float),
                ("norm_eps", c_float), ("n_active", c_int * MAX_LEVELS),
                ("k_cols", c_int * MAX_LEVELS), ("bits", c_int * MAX_LEVELS), ("mode", c_int),
                ("token_stat", c_int), ("col_stat", c_int)]


class FlLayerWeights(ctypes.Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p), ("w_gu", c_void_p), ("w_down", c_void_p),
                ("norm1", c_void_p), ("norm2", c_void_p)]


class FlLayerState(ctypes.Structure):
    _fields_ = [("cache", FlKvCache), ("q_state", c_void_p), ("out", c_void_p), ("lse", c_void_p),
                ("mass_u", c_void_p), ("out_u", c_void_p), ("sel", c_void_p * MAX_LEVELS),
                ("sel_used", c_void_p * MAX_LEVELS), ("k_cur", c_int * MAX_LEVELS),
                ("col_stat", c_void_p * MAX_LEVELS), ("k_in", c_void_p), ("v_in", c_void_p)]


class FlBlockState(ctypes.Structure):
    _fields_ = [("h", c_void_p), ("h_entry", c_void_p), ("active", c_void_p * MAX_LEVELS),
                ("slot", c_void_p * MAX_LEVELS), ("stat", c_void_p),
                ("layers", POINTER(FlLayerState))]


class FlDecodeCfg(ctypes.Structure):
    _fields_ = [("B", c_int), ("N", c_int), ("H", c_int), ("d", c_int), ("g", c_int), ("R", c_int),
                ("n_sink", c_int), ("k_cols", c_int * MAX_LEVELS), ("N_cap", c_int),
                ("rows_cap", c_int * MAX_LEVELS), ("key_group_origin", c_int * MAX_LEVELS)]


class FlDecodeWindow(ctypes.Structure):
    _fields_ = [("cap", c_int), ("count", c_int), ("start", c_int), ("k", c_void_p * MAX_LEVELS),
                ("v", c_void_p * MAX_LEVELS)]


class FlDecodeState(ctypes.Structure):
    _fields_ = [("cache", FlKvCache), ("out", c_void_p), ("lse", c_void_p), ("mass_u", c_void_p),
                ("out_u", c_void_p), ("sel", c_void_p * MAX_LEVELS),
                ("sel_used", c_void_p * MAX_LEVELS), ("k_cur", c_int * MAX_LEVELS),
                ("col_stat", c_void_p * MAX_LEVELS)]


class FlDecodeInputs(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("k_self", c_void_p), ("v_self", c_void_p), ("q_prev", c_void_p),
                ("k_self_prev", c_void_p), ("v_self_prev", c_void_p),
                ("win", POINTER(FlDecodeWindow))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_attention_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.fl_last_error.restype = ctypes.c_char_p
        L.fl_version.restype = ctypes.c_char_p
        L.fl_workspace_size.restype = c_size_t
        L.fl_workspace_size.argtypes = [c_int, c_long, c_long, c_long, c_long]
        L.fl_select_active.argtypes = [c_int, c_int, c_void_p, c_void_p, c_int, c_int, c_void_p, c_int,
                                       c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_size_t, c_void_p]
        L.fl_select_columns.argtypes = [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p,
                                        c_void_p, c_size_t, c_void_p]
        L.fl_kv_residual_quant.argtypes = [POINTER(FlKvCache), c_int, c_int, c_void_p, c_void_p,
                                           c_int, c_void_p]
        L.fl_sparse_loop_attn.argtypes = [POINTER(FlKvCache), POINTER(FlAttnArgs), c_void_p,
                                          c_size_t, c_void_p]
        L.fl_sparse_loop_attn_noalloc.argtypes = [POINTER(FlKvCache), POINTER(FlAttnArgs), c_void_p]
        L.fl_loop_step.argtypes = [POINTER(FlLoopCfg), POINTER(FlLoopState), POINTER(FlLoopInputs),
                                   c_int, c_void_p, c_size_t, c_void_p]
        L.fl_block_step.argtypes = [POINTER(FlBlockCfg), POINTER(FlLayerWeights),
                                    POINTER(FlBlockState), c_int, c_void_p, c_size_t, c_void_p]
        L.fl_decode_step.argtypes = [POINTER(FlDecodeCfg), POINTER(FlDecodeState),
                                     POINTER(FlDecodeInputs), c_int, c_void_p]
        L.fl_sq_err.argtypes = [c_void_p, c_void_p, c_long, c_void_p, c_void_p, c_size_t, c_void_p]
        L.fl_decode_append.argtypes = [POINTER(FlDecodeCfg), POINTER(FlDecodeState),
                                       POINTER(FlDecodeWindow), c_int, c_int, c_void_p]
        L.fl_kv_dequant.argtypes = [POINTER(FlKvCache), c_int, c_int, c_void_p, c_void_p]
        L.fl_timing_enable.argtypes = [c_int]
        L.fl_timing_report.argtypes = [ctypes.c_char_p, c_size_t]
        L.fl_check_indices.argtypes = [c_void_p, c_long, c_long, c_long]
        L.fl_check_finite.argtypes = [c_void_p, c_long]
        L.fl_set_checks.argtypes = [c_int]
        for name in EXPORTS:
            if name not in ("fl_last_error", "fl_version", "fl_workspace_size"):
                getattr(L, name).restype = c_int
        _lib = L
    return _lib


def _p(t):
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream


def _check(fn, rc):
    if rc != 0:
        raise FlError(fn, rc, lib().fl_last_error().decode())


def _dtype_code(t):
    return FL_BF16 if t.dtype == torch.bfloat16 else FL_F32


def fl_version():
    return lib().fl_version().decode()


def fl_workspace_size(op, a, b=0, c=0, e=0):
    return int(lib().fl_workspace_size(op, a, b, c, e))


def fl_timing_enable(level=1):
    """0 off; 1 per-kernel and per-phase events; 2 per-phase events only
    (see the header).  True / False mean 1 / 0."""
    _check("fl_timing_enable", lib().fl_timing_enable(int(level)))


def fl_timing_report():
    """{kernel name: (launches, total ms)} of the launches recorded since the
    last report (waits for their events)."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check("fl_timing_report", lib().fl_timing_report(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


def fl_select_active(h_cur, h_prev, cand, n_select, stat_out, active_out, slot_out=None,
                     stat_in=None, N=None, stat_kind=FL_TOKEN_STAT_ABS, stream=None):
    """Sec. 4.1: token statistic over candidates and nested top-k (see header)."""
    if stat_in is not None:
        n_cand = stat_in.numel()
        dt, D = FL_F32, 0
        N = N if N is not None else (slot_out.numel() if slot_out is not None else n_cand)
    else:
        N, D = h_cur.shape
        dt = _dtype_code(h_cur)
        n_cand = N if cand is None else cand.numel()
    rc = lib().fl_select_active(dt, stat_kind, _p(h_cur), _p(h_prev), N, D, _p(cand), n_cand,
                                n_select,
                                _p(stat_in), _p(stat_out), _p(active_out), _p(slot_out), None, 0,
                                _stream(stream))
    _check("fl_select_active", rc)


def fl_select_columns(col_stat, cand_cols, n_sink, k, sel_out, stream=None):
    """Sec. 4.2: per-head nested column selection with sinks (see header)."""
    H, n_cand = col_stat.shape
    rc = lib().fl_select_columns(_p(col_stat), _p(cand_cols), H, n_cand, n_sink, k, _p(sel_out),
                                 None, 0, _stream(stream))
    _check("fl_select_columns", rc)


def fl_kv_residual_quant(cache: FlKvCache, level, k_new, v_new, gathered=False, stream=None):
    """Sec. 3.3/4.3: writes codes and scales of cache.level[level]."""
    rc = lib().fl_kv_residual_quant(ctypes.byref(cache), level, _dtype_code(k_new), _p(k_new),
                                    _p(v_new), int(gathered), _stream(stream))
    _check("fl_kv_residual_quant", rc)


def fl_sparse_loop_attn(cache: FlKvCache, args: FlAttnArgs, ws, stream=None):
    """Sec. 4.2: sparse attention (+ cache rebuild, + column statistics)."""
    rc = lib().fl_sparse_loop_attn(ctypes.byref(cache), ctypes.byref(args), _p(ws),
                                   ws.numel() * ws.element_size(), _stream(stream))
    _check("fl_sparse_loop_attn", rc)


def fl_sparse_loop_attn_noalloc(cache: FlKvCache, args: FlAttnArgs, stream=None):
    """fl_sparse_loop_attn with the library's per-GPU scratch as workspace
    (allocates nothing; see the header for the size limit and sharing)."""
    rc = lib().fl_sparse_loop_attn_noalloc(ctypes.byref(cache), ctypes.byref(args), _stream(stream))
    _check("fl_sparse_loop_attn_noalloc", rc)


NOALLOC_SCRATCH_BYTES = 80 << 20


def fl_loop_step(cfg: FlLoopCfg, state: FlLoopState, inputs: FlLoopInputs, r, ws, stream=None):
    """Sec. 4.1-4.3: one whole loop r."""
    rc = lib().fl_loop_step(ctypes.byref(cfg), ctypes.byref(state), ctypes.byref(inputs), r,
                            _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("fl_loop_step", rc)


def fl_block_step(cfg: FlBlockCfg, weights, state: FlBlockState, r, ws, stream=None):
    """Sec. 4.1/4.4: one loop r of the whole looped block (all layers)."""
    rc = lib().fl_block_step(ctypes.byref(cfg), weights, ctypes.byref(state), r, _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream))
    _check("fl_block_step", rc)


def fl_decode_step(cfg: FlDecodeCfg, state: FlDecodeState, inputs: FlDecodeInputs, r, stream=None):
    """Sec. 4.2 for one new token per sequence: loop r of batched decode."""
    rc = lib().fl_decode_step(ctypes.byref(cfg), ctypes.byref(state), ctypes.byref(inputs), r,
                              _stream(stream))
    _check("fl_decode_step", rc)


def fl_decode_append(cfg: FlDecodeCfg, state: FlDecodeState, win: FlDecodeWindow, slot, n=1,
                     stream=None):
    """Sec. 4.3 / App. E during generation: append the n tokens in window
    slots slot .. slot + n - 1 (mod the ring) to every sequence's cache (cfg.N
    and the level row counts grow by n; n = g under the asymmetric scheme)."""
    _check("fl_decode_append", lib().fl_decode_append(ctypes.byref(cfg), ctypes.byref(state),
                                                      ctypes.byref(win), slot, n, _stream(stream)))


def fl_kv_dequant(cache: FlKvCache, level, which, out, stream=None):
    """Sec. 3.3 / App. E: fp32 reconstruction [N][H][d] of keys (which=0) or
    values (1) at loop level+1."""
    _check("fl_kv_dequant", lib().fl_kv_dequant(ctypes.byref(cache), level, which, _p(out),
                                                _stream(stream)))


def fl_check_indices(idx, lo, hi):
    """Host-side validation of an index list (numpy int32): strictly
    ascending, every element in [lo, hi); returns (status, message)."""
    import numpy as np
    a = np.ascontiguousarray(idx, dtype=np.int32)
    rc = lib().fl_check_indices(a.ctypes.data_as(c_void_p), a.size, int(lo), int(hi))
    return rc, lib().fl_last_error().decode() if rc else ""


def fl_check_finite(x):
    """Host-side validation of fp32 values (numpy): all finite; returns
    (status, message)."""
    import numpy as np
    a = np.ascontiguousarray(x, dtype=np.float32)
    rc = lib().fl_check_finite(a.ctypes.data_as(c_void_p), a.size)
    return rc, lib().fl_last_error().decode() if rc else ""


def fl_set_checks(on=True):
    """Check mode: entry points validate their device index lists and
    statistics on the host before enqueuing anything (see the header)."""
    _check("fl_set_checks", lib().fl_set_checks(int(bool(on))))


def fl_sq_err(x, ref, out, ws=None, stream=None):
    """App. E calibration error: out[0] = sum (x - ref)^2, out[1] = sum ref^2
    (fp64 device tensor of 2) over two fp32 device tensors of equal size."""
    n = x.numel()
    assert ref.numel() == n and out.dtype == torch.float64 and out.numel() >= 2
    if ws is None:
        ws = torch.empty(fl_workspace_size(FL_WS_SQ_ERR, n), dtype=torch.uint8, device=x.device)
    _check("fl_sq_err", lib().fl_sq_err(_p(x), _p(ref), n, _p(out), _p(ws), ws.numel(),
                                        _stream(stream)))


# --------------------------------------------------------------------------
# Device-memory holder for a whole R-loop run (buffers only; no arithmetic).

def level_code_bytes(bits, H, d):
    return H * d * bits // 8


def alloc_level(L, rows, H, d, g, bits, scheme, buf):
    """Allocate one cache level's codes, scales (and offsets under the
    asymmetric scheme) with ``buf(shape, dtype)`` and point descriptor L at
    them; returns the tensors."""
    kc = buf((rows, H, d * bits // 8), torch.uint8)
    vc = buf((rows, H, d * bits // 8), torch.uint8)
    vshape = (rows, H, d // g)
    kshape = ((rows + g - 1) // g, H, d) if scheme == FL_QUANT_ASYM else vshape
    t = dict(k=kc, v=vc, ks=buf(kshape, torch.float32), vs=buf(vshape, torch.float32))
    if scheme == FL_QUANT_ASYM:
        t["kz"] = buf(kshape, torch.float32)
        t["vz"] = buf(vshape, torch.float32)
    L.bits, L.n_rows = bits, rows
    L.k_codes, L.v_codes, L.k_scale, L.v_scale = _p(kc), _p(vc), _p(t["ks"]), _p(t["vs"])
    L.k_zero, L.v_zero = _p(t.get("kz")), _p(t.get("vz"))
    return t


class LoopRunner:
    """Allocates the cache levels and loop state for one attention layer of
    N tokens and runs ``fl_loop_step`` for r = 1..R."""

    def __init__(self, N, H, d, g, R, n_sink, n_active, k_cols, bits, dtype=torch.bfloat16,
                 mode=FL_DEQ_AUTO, token_stat=FL_TOKEN_STAT_ABS, col_stat=FL_COL_STAT_MASS,
                 quant=FL_QUANT_ABSMAX, device="cuda"):
        self.N, self.H, self.d, self.g, self.R = N, H, d, g, R
        dev = torch.device(device)
        self.dev = dev
        cfg = FlLoopCfg()
        cfg.N, cfg.H, cfg.d, cfg.g, cfg.R, cfg.n_sink = N, H, d, g, R, n_sink
        cfg.dtype = FL_BF16 if dtype == torch.bfloat16 else FL_F32
        cfg.mode = mode
        cfg.token_stat, cfg.col_stat = token_stat, col_stat
        for r in range(R):
            cfg.n_active[r] = n_active[r]
            cfg.k_cols[r] = k_cols[r]
            cfg.bits[r] = bits[r]
        self.cfg = cfg
        st = FlLoopState()
        self._keep = []

        def buf(shape, dt):
            t = torch.empty(shape, dtype=dt, device=dev)
            self._keep.append(t)
            return t

        st.cache.N, st.cache.H, st.cache.d, st.cache.g = N, H, d, g
        st.cache.scheme = quant
        # per-token operand classes (written by the quantiser, read by the attention)
        self.cls = buf((2, N, H), torch.uint8)
        st.cache.cls = _p(self.cls)
        self.codes = []
        for r in range(R):
            rows = N if r == 0 else n_active[r]
            self.codes.append(alloc_level(st.cache.level[r], rows, H, d, g, bits[r], quant, buf))
        self.active, self.slot, self.sel, self.col_stat = [], [], [], []
        for r in range(R):
            a = buf((n_active[r],), torch.int32)
            s = buf((N,), torch.int32) if r > 0 else None
            sl = buf((H, k_cols[r]), torch.int32) if r > 0 and k_cols[r] < N else None
            k_here = min(k_cols[: r + 1])
            cs = buf((H, k_here), torch.float32)
            st.active[r] = _p(a)
            st.slot[r] = _p(s)
            st.sel[r] = _p(sl)
            st.col_stat[r] = _p(cs)
            self.active.append(a); self.slot.append(s); self.sel.append(sl); self.col_stat.append(cs)
        self.stat = buf((N,), torch.float32)
        self.out = buf((N, H, d), torch.float32)
        self.lse = buf((N, H), torch.float32)
        self.mass_u = buf((N, H), torch.float32)
        self.out_u = buf((N, H, d), torch.float32)
        st.stat, st.out, st.lse = _p(self.stat), _p(self.out), _p(self.lse)
        st.mass_u, st.out_u = _p(self.mass_u), _p(self.out_u)
        self.state = st
        ws_bytes = fl_workspace_size(FL_WS_LOOP_STEP, H, N, d, R)
        self.ws = buf((ws_bytes,), torch.uint8)
        self.inputs = FlLoopInputs()

    def step(self, r, h_cur, h_prev, q, k, v, q_prev, stream=None):
        inp = self.inputs
        inp.h_cur, inp.h_prev = _p(h_cur), _p(h_prev)
        inp.q, inp.k, inp.v, inp.q_prev = _p(q), _p(k), _p(v), _p(q_prev)
        fl_loop_step(self.cfg, self.state, inp, r, self.ws, stream)

    def sel_used(self, r):
        """Column set used at loop r (None = all columns)."""
        p = self.state.sel_used[r - 1]
        if not p:
            return None
        for t in self.sel:
            if t is not None and t.data_ptr() == p:
                return t
        raise RuntimeError("unknown selection buffer")

    def k_used(self, r):
        return self.state.k_cur[r - 1]

    # ---- checkpoint / resume of the loop state ----
    def _state_tensors(self):
        """Every device buffer that carries state from one loop to the next
        (the workspace is scratch and carries none)."""
        named = {}
        for r, lev in enumerate(self.codes):
            for key, t in lev.items():
                named[f"level{r}.{key}"] = t
        for r in range(self.R):
            for key in ("active", "slot", "sel", "col_stat"):
                t = getattr(self, key)[r]
                if t is not None:
                    named[f"{key}{r}"] = t
        for key in ("stat", "out", "lse", "mass_u", "out_u", "cls"):
            named[key] = getattr(self, key)
        return named

    def snapshot(self):
        """Host copy of the whole loop state after some loop: the device
        buffers of the cache levels and per-loop state, and the host-side
        bookkeeping of fl_loop_state (column counts, which selection each loop
        used, the cache levels' row counts and widths).  ``restore`` on a
        runner of the same configuration (this one or a fresh one) resumes
        from it."""
        torch.cuda.synchronize()
        st = self.state
        sel_idx = []
        for r in range(self.R):
            p = st.sel_used[r]
            sel_idx.append(None if not p else
                           next(i for i, t in enumerate(self.sel) if t is not None and t.data_ptr() == p))
        levels = [(st.cache.level[r].bits, st.cache.level[r].n_rows, bool(st.cache.level[r].rows))
                  for r in range(self.R)]
        return dict(tensors={k: t.cpu().clone() for k, t in self._state_tensors().items()},
                    k_cur=[st.k_cur[r] for r in range(self.R)], sel_used=sel_idx, levels=levels,
                    n_levels=st.cache.n_levels)

    def restore(self, snap):
        mine = self._state_tensors()
        assert set(mine) == set(snap["tensors"]), "snapshot of another configuration"
        for k, t in mine.items():
            t.copy_(snap["tensors"][k])
        st = self.state
        for r in range(self.R):
            st.k_cur[r] = snap["k_cur"][r]
            i = snap["sel_used"][r]
            st.sel_used[r] = None if i is None else self.sel[i].data_ptr()
            bits, n_rows, has_rows = snap["levels"][r]
            L = st.cache.level[r]
            L.bits, L.n_rows = bits, n_rows
            L.rows = st.active[r] if has_rows else None
            L.slot = st.slot[r] if has_rows else None
        st.cache.n_levels = snap["n_levels"]
        torch.cuda.synchronize()


class BlockRunner:
    """Allocates per-layer caches and state for the looped block and runs
    ``fl_block_step`` for r = 1..R.  ``weights`` is a list (one per layer) of
    dicts of bf16 device tensors: w_qkv [3D][D], w_o [D][D], w_gu [2F][D]
    (rows 2j gate, 2j+1 up), w_down [D][F], norm1 [D], norm2 [D]."""

    def __init__(self, N, H, d, g, R, n_sink, n_active, k_cols, bits, weights, ffn,
                 rope_theta=10000.0, norm_eps=1e-6, mode=FL_DEQ_AUTO,
                 token_stat=FL_TOKEN_STAT_ABS, col_stat=FL_COL_STAT_MASS, row_capacity=None,
                 quant=FL_QUANT_ABSMAX, capture_kv=False, device="cuda"):
        """row_capacity: per-loop row counts to allocate (default n_active),
        so that ``set_active_counts`` can later run other schedules.
        capture_kv: also keep each layer's latest pre-quantisation keys (after
        RoPE) and values of the active rows (``layer_bufs[l]["k_in"]``,
        ``["v_in"]``, bf16 [N][H][d], first n_active rows valid)."""
        dev = torch.device(device)
        self.N, self.H, self.d, self.R, self.g = N, H, d, R, g
        cap = list(row_capacity) if row_capacity is not None else list(n_active)
        self.cap = cap
        self.L = len(weights)
        D = H * d
        self._keep = []

        def buf(shape, dt):
            t = torch.empty(shape, dtype=dt, device=dev)
            self._keep.append(t)
            return t

        cfg = FlBlockCfg()
        cfg.N, cfg.H, cfg.d, cfg.g, cfg.R, cfg.n_sink = N, H, d, g, R, n_sink
        cfg.n_layers, cfg.ffn, cfg.rope_theta, cfg.norm_eps, cfg.mode = self.L, ffn, rope_theta, norm_eps, mode
        cfg.token_stat, cfg.col_stat = token_stat, col_stat
        for r in range(R):
            cfg.n_active[r], cfg.k_cols[r], cfg.bits[r] = n_active[r], k_cols[r], bits[r]
        self.cfg = cfg
        W = (FlLayerWeights * self.L)()
        for l, wd in enumerate(weights):
            for key in ("w_qkv", "w_o", "w_gu", "w_down", "norm1", "norm2"):
                setattr(W[l], key, _p(wd[key]))
        self.W = W
        self.weights = weights
        layers = (FlLayerState * self.L)()
        self.layer_bufs = []
        for l in range(self.L):
            Ls = layers[l]
            Ls.cache.N, Ls.cache.H, Ls.cache.d, Ls.cache.g = N, H, d, g
            Ls.cache.scheme = quant
            lb = dict(codes=[])
            lb["cls"] = buf((2, N, H), torch.uint8)
            Ls.cache.cls = _p(lb["cls"])
            for r in range(R):
                rows = N if r == 0 else cap[r]
                lb["codes"].append(alloc_level(Ls.cache.level[r], rows, H, d, g, bits[r], quant,
                                               buf))
            lb["q_state"] = buf((N, H, d), torch.bfloat16)
            lb["out"] = buf((N, H, d), torch.float32)
            lb["lse"] = buf((N, H), torch.float32)
            lb["mass_u"] = buf((N, H), torch.float32)
            lb["out_u"] = buf((N, H, d), torch.float32)
            Ls.q_state, Ls.out, Ls.lse = _p(lb["q_state"]), _p(lb["out"]), _p(lb["lse"])
            Ls.mass_u, Ls.out_u = _p(lb["mass_u"]), _p(lb["out_u"])
            if capture_kv:
                lb["k_in"] = buf((N, H, d), torch.bfloat16)
                lb["v_in"] = buf((N, H, d), torch.bfloat16)
                Ls.k_in, Ls.v_in = _p(lb["k_in"]), _p(lb["v_in"])
            lb["sel"], lb["col_stat"] = [], []
            for r in range(R):
                sl = buf((H, k_cols[r]), torch.int32) if r > 0 and k_cols[r] < N else None
                cs = buf((H, min(k_cols[: r + 1])), torch.float32)
                Ls.sel[r] = _p(sl)
                Ls.col_stat[r] = _p(cs)
                lb["sel"].append(sl); lb["col_stat"].append(cs)
            self.layer_bufs.append(lb)
        self.layers = layers
        st = FlBlockState()
        self.h = buf((N, D), torch.float32)
        self.h_entry = buf((N, D), torch.float32)
        self.stat = buf((N,), torch.float32)
        self.active, self.slot = [], []
        for r in range(R):
            a = buf((cap[r],), torch.int32)
            s_ = buf((N,), torch.int32) if r > 0 else None
            st.active[r], st.slot[r] = _p(a), _p(s_)
            self.active.append(a); self.slot.append(s_)
        st.h, st.h_entry, st.stat = _p(self.h), _p(self.h_entry), _p(self.stat)
        st.layers = ctypes.cast(layers, POINTER(FlLayerState))
        self.state = st
        self.ws = buf((fl_workspace_size(FL_WS_BLOCK_STEP, N, H, d, ffn),), torch.uint8)

    def step(self, r, stream=None):
        fl_block_step(self.cfg, self.W, self.state, r, self.ws, stream)

    def set_active_counts(self, n_active):
        """Use another nested schedule of active-row counts (within the
        allocated capacity); takes effect from the next loop 1."""
        assert len(n_active) == self.R and n_active[0] == self.N
        for r in range(1, self.R):
            if not 1 <= n_active[r] <= min(n_active[r - 1], self.cap[r]):
                raise ValueError(f"n_active[{r}] = {n_active[r]} outside [1, "
                                 f"{min(n_active[r - 1], self.cap[r])}]")
        for r in range(self.R):
            self.cfg.n_active[r] = n_active[r]


class DecodeRunner:
    """Batched-decode buffers: B sequences' loop-indexed prefix caches (one
    allocation per level, sequences back to back as ``fl_decode_step``
    expects) and the new tokens' per-loop state.  ``load_sequence`` fills
    sequence b's cache through the library (``fl_select_active`` on the given
    statistic, ``fl_kv_residual_quant`` per level); ``step`` runs loop r."""

    def __init__(self, B, N, H, d, g, R, n_sink, n_active, k_cols, bits, gen_tokens=0, window=64,
                 quant=FL_QUANT_ABSMAX, device="cuda"):
        """gen_tokens > 0 prepares generation: caches with room for that many
        appended positions and per-loop bf16 window rings of window + F slots
        (the window, the tokens waiting to leave it together and the token
        being decoded); tokens leave the window F at a time, F = 1 under the
        absmax scheme and F = g under FL_QUANT_ASYM (the paper's quantiser,
        whose keys are quantised per channel over g rows: each appended block
        is a key group of its own, from the prompt's sizes on)."""
        dev = torch.device(device)
        self.B, self.N, self.H, self.d, self.g, self.R = B, N, H, d, g, R
        self.quant = quant
        self.n_active, self.k_cols, self.bits = list(n_active), list(k_cols), list(bits)
        self.gen_tokens, self.window = gen_tokens, window
        self.flush = g if quant == FL_QUANT_ASYM else 1
        self._keep = []

        def buf(shape, dt):
            t = torch.empty(shape, dtype=dt, device=dev)
            self._keep.append(t)
            return t

        cfg = FlDecodeCfg()
        cfg.B, cfg.N, cfg.H, cfg.d, cfg.g, cfg.R, cfg.n_sink = B, N, H, d, g, R, n_sink
        for r in range(R):
            cfg.k_cols[r] = k_cols[r]
        cap_pos = N + gen_tokens
        if gen_tokens:
            cfg.N_cap = cap_pos
            for r in range(1, R):
                cfg.rows_cap[r] = n_active[r] + gen_tokens
            if quant == FL_QUANT_ASYM:
                for r in range(R):
                    cfg.key_group_origin[r] = N if r == 0 else n_active[r]
        self.cfg = cfg
        st = FlDecodeState()
        C = st.cache
        C.N, C.H, C.d, C.g, C.n_levels, C.scheme = N, H, d, g, R, quant
        self.codes, self.rows, self.slot = [], [], []
        for r in range(R):
            n = N if r == 0 else n_active[r]
            nc = cap_pos if r == 0 else n + gen_tokens
            cb = dict(k=buf((B, nc, H, d * bits[r] // 8), torch.uint8),
                      v=buf((B, nc, H, d * bits[r] // 8), torch.uint8),
                      vs=buf((B, nc, H, d // g), torch.float32))
            if quant == FL_QUANT_ASYM:
                # keys: a scale and offset per channel for every g rows, the
                # appended rows in groups of their own from the origin on
                o = cfg.key_group_origin[r]
                ng = (o + g - 1) // g + (nc - o + g - 1) // g
                cb.update(ks=buf((B, ng, H, d), torch.float32), kz=buf((B, ng, H, d), torch.float32),
                          vz=buf((B, nc, H, d // g), torch.float32))
            else:
                cb["ks"] = buf((B, nc, H, d // g), torch.float32)
            # row lists and slot maps start as -1 (no row) beyond what is filled
            rows = buf((B, nc), torch.int32).fill_(-1) if r > 0 else None
            slot = buf((B, cap_pos), torch.int32).fill_(-1) if r > 0 else None
            Lv = C.level[r]
            Lv.bits, Lv.n_rows = bits[r], n
            Lv.rows, Lv.slot = _p(rows), _p(slot)
            Lv.k_codes, Lv.v_codes, Lv.k_scale, Lv.v_scale = _p(cb["k"]), _p(cb["v"]), _p(cb["ks"]), _p(cb["vs"])
            Lv.k_zero, Lv.v_zero = _p(cb.get("kz")), _p(cb.get("vz"))
            self.codes.append(cb); self.rows.append(rows); self.slot.append(slot)
        self.out = buf((B, H, d), torch.float32)
        self.lse = buf((B, H), torch.float32)
        self.mass_u = buf((B, H), torch.float32)
        self.out_u = buf((B, H, d), torch.float32)
        st.out, st.lse, st.mass_u, st.out_u = _p(self.out), _p(self.lse), _p(self.mass_u), _p(self.out_u)
        self.sel, self.col_stat = [], []
        # budgets with loop 1 at the largest context the cache can reach
        kce = [cap_pos] + list(k_cols[1:])
        for r in range(R):
            sl = buf((B, H, k_cols[r]), torch.int32) if r > 0 and k_cols[r] < min(kce[:r]) else None
            cs = buf((B, H, min(kce[: r + 1])), torch.float32)
            st.sel[r], st.col_stat[r] = _p(sl), _p(cs)
            self.sel.append(sl); self.col_stat.append(cs)
        self.state = st
        self.win = None
        if gen_tokens:
            wn = FlDecodeWindow()
            wn.cap, wn.count, wn.start = window + self.flush, 0, 0
            self.win_k = [buf((B, wn.cap, H, d), torch.bfloat16) for _ in range(R)]
            self.win_v = [buf((B, wn.cap, H, d), torch.bfloat16) for _ in range(R)]
            for r in range(R):
                wn.k[r], wn.v[r] = _p(self.win_k[r]), _p(self.win_v[r])
            self.win = wn
            self.t = 0

    def seq_cache(self, b):
        """FlKvCache of sequence b alone (pointers into the batched buffers)."""
        c = FlKvCache()
        c.N, c.H, c.d, c.g, c.n_levels, c.scheme = self.N, self.H, self.d, self.g, self.R, self.quant
        for r in range(self.R):
            Lv = c.level[r]
            cb = self.codes[r]
            Lv.bits, Lv.n_rows = self.bits[r], (self.N if r == 0 else self.n_active[r])
            Lv.rows = None if r == 0 else _p(self.rows[r][b])
            Lv.slot = None if r == 0 else _p(self.slot[r][b])
            Lv.k_codes, Lv.v_codes = _p(cb["k"][b]), _p(cb["v"][b])
            Lv.k_scale, Lv.v_scale = _p(cb["ks"][b]), _p(cb["vs"][b])
            if "kz" in cb:
                Lv.k_zero, Lv.v_zero = _p(cb["kz"][b]), _p(cb["vz"][b])
        return c

    def load_sequence(self, b, k, v, stat, stream=None):
        """k, v: per-loop bf16 device tensors [N][H][d] of the prefix tokens;
        stat: per-loop fp32 device tensors [N] (stat[0] unused)."""
        c = self.seq_cache(b)
        for r in range(self.R):
            if r > 0:
                # the previous loop's active rows (the buffer may have room for more)
                cand = None if r == 1 else self.rows[r - 1][b][: self.n_active[r - 1]]
                key = stat[r] if cand is None else stat[r].index_select(0, cand.long())
                fl_select_active(None, None, cand, self.n_active[r], None, self.rows[r][b],
                                 self.slot[r][b], stat_in=key, N=self.N, stream=stream)
            fl_kv_residual_quant(c, r, k[r], v[r], gathered=False, stream=stream)
        self._cache_views = c

    def step(self, r, q, k_self, v_self, q_prev=None, k_prev=None, v_prev=None, stream=None):
        inp = FlDecodeInputs()
        inp.q, inp.k_self, inp.v_self = _p(q), _p(k_self), _p(v_self)
        inp.q_prev, inp.k_self_prev, inp.v_self_prev = _p(q_prev), _p(k_prev), _p(v_prev)
        fl_decode_step(self.cfg, self.state, inp, r, stream)

    def generate(self, q, k, v, stream=None, after_loop=None):
        """Decode the next generated token of every sequence through all R
        loops.  q, k, v: lists of R bf16 device tensors [B][H][d].  When the
        ring is full, its oldest F tokens are appended to the cache first and
        leave it; this token's K/V then take the next free slot."""
        win, t = self.win, self.t
        if win.count == win.cap:
            fl_decode_append(self.cfg, self.state, win, win.start, self.flush, stream)
            win.start = (win.start + self.flush) % win.cap
            win.count -= self.flush
        slot = (win.start + win.count) % win.cap
        for r in range(self.R):
            self.win_k[r][:, slot].copy_(k[r])
            self.win_v[r][:, slot].copy_(v[r])
        win.count += 1
        inp = FlDecodeInputs()
        inp.win = ctypes.pointer(win)
        for r in range(1, self.R + 1):
            inp.q = _p(q[r - 1])
            inp.q_prev = _p(q[r - 2]) if r > 1 else None
            fl_decode_step(self.cfg, self.state, inp, r, stream)
            if after_loop is not None:
                after_loop(r)
        self.t = t + 1

    def k_used(self, r):
        return self.state.k_cur[r - 1]

    def sel_used(self, r):
        """Selected prefix columns of loop r ([B][H][k]) or None (dense)."""
        p = self.state.sel_used[r - 1]
        if not p:
            return None
        for t in self.sel:
            if t is not None and t.data_ptr() == p:
                return t
        raise RuntimeError("unknown selection buffer")
