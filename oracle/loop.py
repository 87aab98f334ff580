"""Whole-loop driver of the oracle: chains the fp32 step functions of
``flo_oracle.c`` in the order the FlashLoop paper applies them.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Per loop r (paper Sec. 4.1-4.3; the first loop is dense, Sec. 4.1 "after the
dense early loops"):

  loop 1   base-quantise K_1, V_1; dense causal attention on the dequantised
           cache; column statistics of every column; A_1 = all tokens,
           S_1 = all columns, M_U = O_U = 0.
  loop r   (1) token statistic ||h_r - h_{r-1}|| (or its ratio to
               ||h_{r-1}||) over A_{r-1};
           (2) A_r = top n_r of A_{r-1};
           (3) residual level r-1 for rows A_r against the dequantised
               previous loop; other rows keep their previous K/V;
           (4) S_r = sinks + top (k_r - sinks) of S_{r-1} by c_{r-1}
               (S_r = S_{r-1} when it already fits k_r);
           (5) when S_r != S_{r-1}: pruned-column caches M_U / O_U under loop
               r-1's distribution, else carried;
           (6) sparse attention of A_r over S_r(i);
           (7) column statistics c_r when the next loop prunes further.

Optional ``override`` hooks let a test feed the GPU's own fp32 statistic
buffers into the oracle's selection, so index sets are compared from the same
inputs (a selection that is unique given those buffers).
"""
from __future__ import annotations

import numpy as np

from . import (active_count, attend, column_stats, delta_norm, quantize_rows, quantize_rows_asym,
               select_columns, top_select, unselected_cache)


def _level(xnew, xprev, g, bits, asym=False, per_channel=False):
    """One cache level: the spec's absmax quantiser, or (asym) the paper's
    App. E min/max quantiser with keys per channel and values per token."""
    if asym:
        codes, scales, zeros, xhat = quantize_rows_asym(xnew, xprev, g, bits, per_channel)
        return dict(codes=codes, scales=scales, zeros=zeros, raw=None), xhat
    codes, scales, raw, xhat = quantize_rows(xnew, xprev, g, bits)
    return dict(codes=codes, scales=scales, raw=raw), xhat


def run_prefill(h, q, k, v, sched, override=None, stats_every_loop=False,
                keep_dense=False):
    """Run loops 1..R of the lazy-update attention step.

    h: list of R arrays [N][D]; q, k, v: lists of R arrays [N][H][d] (fp32
    values; bf16 inputs are passed as their exact fp32 expansion).
    sched: dict with N, H, d, g, R, n_sink, rho[R], kcols[R], bits[R]
    (bits[0] is the base level: 8 or 32); optional token_stat "abs" (default)
    or "rel" (normalised change, Sec. 4.1) and col_stat "mass" (default) or
    "vnorm" (mass weighted by the column's value norm, Sec. 4.2); optional
    quant "absmax" (default, the spec's quantiser) or "asym" (App. E: min/max
    with scale and offset, keys per channel over g packed rows, values per
    token).
    override: optional dict {('stat', r): array, ('cstat', r): array} used in
    place of the oracle's own statistic for the selection made at loop r.
    Returns a list of per-loop dicts.
    """
    override = override or {}
    N, H, d, g, R = (sched[x] for x in ("N", "H", "d", "g", "R"))
    sm = np.float32(1.0 / np.sqrt(d))
    n_sink = sched["n_sink"]
    out = []

    asym = sched.get("quant", "absmax") == "asym"
    # ---- loop 1: dense ----
    lk, khat = _level(k[0], None, g, sched["bits"][0], asym, True)
    lv, vhat = _level(v[0], None, g, sched["bits"][0], asym, False)
    o1, lse1 = attend(q[0], khat, vhat, None, None, sm)
    need_c = R > 1 and (stats_every_loop or sched["kcols"][1] < N)
    vw = sched.get("col_stat", "mass") == "vnorm"
    rel = sched.get("token_stat", "abs") == "rel"
    c1 = column_stats(q[0], khat, None, None, lse1, sm, vhat=vhat if vw else None) \
        if need_c else None
    A = np.arange(N, dtype=np.int32)
    S = None
    k_cur = N
    o_d = o1.copy(); lse_d = lse1.copy()
    mu_d = np.zeros((N, H), np.float32); ou_d = np.zeros((N, H, d), np.float32)
    rec = dict(r=1, active=A, n=N, level_k=lk, level_v=lv, sel=None, k=N,
               mass_u=np.zeros((N, H), np.float32), out_u=None, out=o1, lse=lse1, cstat=c1)
    if keep_dense:
        rec.update(khat=khat, vhat=vhat)
    out.append(rec)
    cstat = c1

    for r in range(2, R + 1):
        # (1)-(2) token selection, nested in A_{r-1}
        stat = delta_norm(h[r - 1], h[r - 2], cand=A, relative=rel)
        stat_sel = override.get(("stat", r), stat)
        n_r = active_count(sched["rho"][r - 1], N, len(A))
        A_new = top_select(stat_sel, n_r, pos=A)
        # (3) residual level for the active rows
        lk, krows = _level(k[r - 1][A_new], khat[A_new], g, sched["bits"][r - 1], asym, True)
        lv, vrows = _level(v[r - 1][A_new], vhat[A_new], g, sched["bits"][r - 1], asym, False)
        khat_new = khat.copy(); khat_new[A_new] = krows
        vhat_new = vhat.copy(); vhat_new[A_new] = vrows
        # (4) column selection
        k_r = sched["kcols"][r - 1]
        if k_cur <= k_r:
            S_new, k_new, changed = S, k_cur, False
        else:
            cs = override.get(("cstat", r), cstat)
            S_new = select_columns(cs, S, k_r, n_sink)
            k_new, changed = k_r, True
        # (5) caches of pruned columns
        if changed:
            mu, ou = unselected_cache(q[r - 2], khat, vhat, A_new, S, S_new, lse_d[A_new], sm,
                                      None if S is None else mu_d[A_new],
                                      None if S is None else ou_d[A_new])
        else:
            mu, ou = mu_d[A_new].copy(), ou_d[A_new].copy()
        # (6) sparse attention
        o_r, lse_r = attend(q[r - 1], khat_new, vhat_new, A_new, S_new, sm, mu, ou)
        # (7) column statistics for the next selection
        need_c = stats_every_loop or (r < R and sched["kcols"][r] < k_new)
        c_r = column_stats(q[r - 1], khat_new, A_new, S_new, lse_r, sm, mu,
                           vhat=vhat_new if vw else None) if need_c else None
        rec = dict(r=r, stat=stat, active=A_new, n=n_r, level_k=lk, level_v=lv, sel=S_new,
                   k=k_new, sel_changed=changed, mass_u=mu, out_u=ou, out=o_r, lse=lse_r,
                   cstat=c_r)
        if keep_dense:
            rec.update(khat=khat_new, vhat=vhat_new)
        out.append(rec)
        # carry state
        o_d[A_new] = o_r; lse_d[A_new] = lse_r; mu_d[A_new] = mu; ou_d[A_new] = ou
        A, S, k_cur, khat, vhat, cstat = A_new, S_new, k_new, khat_new, vhat_new, c_r
    return out


def dense_output(res, N):
    """Full [N][H][d] output after the last loop: rows inactive in a loop keep
    the output of the last loop that computed them (Sec. 4.1)."""
    o = res[0]["out"].copy()
    for rec in res[1:]:
        o[rec["active"]] = rec["out"]
    return o
