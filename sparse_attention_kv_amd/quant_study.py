"""Residual versus direct quantisation of the per-loop KV cache (FlashLoop
paper, Sec. 3.3 and Fig. 2(c); the "Per-loop KIVI4" ablation of Table 2).

For loop-wise K/V of N tokens (every token active in every loop, as in the
paper's analysis of full KV states) and one quantiser, per loop r:

  residual  the loop-indexed cache: loop 1 quantised directly, every later
            loop as a quantised residual against the previous loop's
            reconstruction; error of the reconstruction at loop r;
  direct    loop r's K/V quantised on their own with the same scheme and
            bit width (one base level);
  update    ||x_r - x_{r-1}|| / ||x_r||, the size of the cross-loop change
            the residual carries (Fig. 3(c,d) plot its decrease with depth).

Errors are relative Frobenius norms over all tokens, heads and channels,
||xhat - x|| / ||x||.  Quantisation, reconstruction and the error sums run in
the library (``fl_kv_residual_quant``, ``fl_kv_dequant``, ``fl_sq_err``);
this module allocates buffers and sequences the calls.
"""
from __future__ import annotations

import math

import torch

from . import fl


class _Cache:
    """A loop-indexed cache of N tokens with every token present in every
    level (buffers only)."""

    def __init__(self, N, H, d, g, bits, scheme, device):
        self._keep = []

        def buf(shape, dt):
            t = torch.zeros(shape, dtype=dt, device=device)
            self._keep.append(t)
            return t

        c = fl.FlKvCache()
        c.N, c.H, c.d, c.g, c.n_levels, c.scheme = N, H, d, g, len(bits), scheme
        rows = torch.arange(N, dtype=torch.int32, device=device)
        self._keep.append(rows)
        for l, b in enumerate(bits):
            fl.alloc_level(c.level[l], N, H, d, g, b, scheme, buf)
            if l > 0:
                c.level[l].rows = rows.data_ptr()
                c.level[l].slot = rows.data_ptr()      # slot of token i is i
        self.cache = c


def _rel(meter, xhat, x):
    fl.fl_sq_err(xhat, x, meter["out"], meter["ws"])
    e2, r2 = meter["out"].tolist()
    return math.sqrt(e2 / r2) if r2 > 0 else 0.0


def residual_vs_direct(ks, vs, g, bits, scheme=fl.FL_QUANT_ASYM):
    """ks, vs: per-loop [N][H][d] device tensors (bf16 or fp32).  bits: per
    loop (index 0 = loop 1's base level).  The direct leg quantises loop r
    with bits[r-1] as a base level of the same scheme (under the absmax
    scheme base levels are int8, so that leg uses 8 bits).
    Returns a list of per-loop dicts with k_res, k_dir, v_res, v_dir,
    k_update, v_update."""
    R = len(ks)
    N, H, d = ks[0].shape
    dev = ks[0].device
    n = N * H * d
    meter = dict(out=torch.zeros(2, dtype=torch.float64, device=dev),
                 ws=torch.empty(fl.fl_workspace_size(fl.FL_WS_SQ_ERR, n), dtype=torch.uint8,
                                device=dev))
    chain = _Cache(N, H, d, g, bits, scheme, dev)
    xhat = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    out = []
    for r in range(1, R + 1):
        k, v = ks[r - 1].contiguous(), vs[r - 1].contiguous()
        fl.fl_kv_residual_quant(chain.cache, r - 1, k, v)
        b_dir = bits[r - 1] if scheme == fl.FL_QUANT_ASYM else 8
        direct = _Cache(N, H, d, g, [b_dir], scheme, dev)
        fl.fl_kv_residual_quant(direct.cache, 0, k, v)
        rec = dict(r=r)
        for which, name, x in ((0, "k", k), (1, "v", v)):
            xf = x.float()
            fl.fl_kv_dequant(chain.cache, r - 1, which, xhat)
            rec[name + "_res"] = _rel(meter, xhat, xf)
            fl.fl_kv_dequant(direct.cache, 0, which, xhat)
            rec[name + "_dir"] = _rel(meter, xhat, xf)
            if r > 1:
                prev = (ks if which == 0 else vs)[r - 2].float()
                rec[name + "_update"] = _rel(meter, prev, xf)
        out.append(rec)
    return out
