"""Oracle of batched decode with the lazy-update loop attention.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

FlashLoop paper, Sec. 4.2-4.3 applied to one new token per sequence (Sec.
5.3.1 evaluates decode).  A sequence has a prefix of N cached tokens whose
cache was built loop by loop as in prefill: loop 1 stores every token's K/V
as the base level; loop r >= 2 keeps the top n_r of the previous loop's
active tokens by their statistic (nested) and stores their residual level
r-1 against the dequantised previous value; the other tokens keep theirs.

The new token at position N runs R loops.  At loop r its query attends
causally to the prefix's loop-r dequantised keys/values on the selected
columns S_r plus its own fresh key/value (column N, always selected) -- and,
during generation, the unquantised window of recent generated tokens (also
always selected; ``run_generation``):

  loop 1   dense over all N + 1 columns; M_U = O_U = 0; the column
           statistic is the token's probability of every prefix column.
  loop r   S_r = sinks + top (k_r - sinks) of S_{r-1} by the previous
           statistic (kept when it already fits k_r); when it changes,
           M_U / O_U of the pruned columns under loop r-1's distribution
           (its query, cache and self column); sparse attention
           o = (1 - M_U) softmax_{S_r + self} + O_U; the statistic is the
           probability of each kept prefix column.

Every step is a call of the pinned C oracle on an (N + 1)-position problem
with one query row at position N.
"""
from __future__ import annotations

import numpy as np

from . import (active_count, attend, column_stats, quantize_rows, quantize_rows_asym, select_columns,
               top_select, unselected_cache)

F32 = np.float32


def build_cache(k, v, stat, sched):
    """Per-loop prefix cache of one sequence.

    k, v: lists of R fp32 arrays [N][H][d] (the prefix tokens' loop-r K/V);
    stat: list of R entries, stat[r-1] [N] the loop-r selection statistic
    (stat[0] unused).  sched["quant"] "asym" takes the paper's quantiser
    (App. E: keys per channel over g consecutive rows of the level, values per
    g channels of a row; the level's rows in ascending position order) instead
    of the spec's absmax one.  Returns a list of per-loop dicts with the active
    set, the level's codes/scales (and, asym, zeros) and the dequantised cache
    khat/vhat [N][H][d]."""
    N, g = sched["N"], sched["g"]
    asym = sched.get("quant", "absmax") == "asym"
    A = np.arange(N, dtype=np.int32)
    khat = vhat = None
    out = []
    for r in range(1, sched["R"] + 1):
        if r > 1:
            n_r = active_count(sched["rho"][r - 1], N, len(A))
            A = top_select(np.asarray(stat[r - 1], F32)[A], n_r, A)
        bits = sched["bits"][r - 1]
        kp = None if r == 1 else khat[A]
        vp = None if r == 1 else vhat[A]
        if asym:
            kc, ks, kz, kx = quantize_rows_asym(np.asarray(k[r - 1], F32)[A], kp, g, bits, True)
            vc, vs, vz, vx = quantize_rows_asym(np.asarray(v[r - 1], F32)[A], vp, g, bits, False)
        else:
            kc, ks, _, kx = quantize_rows(np.asarray(k[r - 1], F32)[A], kp, g, bits)
            vc, vs, _, vx = quantize_rows(np.asarray(v[r - 1], F32)[A], vp, g, bits)
            kz = vz = None
        if r == 1:
            khat, vhat = kx, vx
        else:
            khat = khat.copy(); khat[A] = kx
            vhat = vhat.copy(); vhat[A] = vx
        out.append(dict(active=A, k_codes=kc, k_scale=ks, k_zero=kz, v_codes=vc, v_scale=vs,
                        v_zero=vz, khat=khat, vhat=vhat))
    return out


def _with_tail(sel, N, T):
    """Per-head selected prefix columns plus the T always-included columns
    at positions N .. N+T-1."""
    tail = np.broadcast_to(np.arange(N, N + T, dtype=np.int32), (sel.shape[0], T))
    return np.concatenate([sel, tail], axis=1)


def decode_token(khat, vhat, q, tail_k, tail_v, sched, override=None):
    """Loops 1..R of one new token over a prefix cache plus bf16 columns.

    khat, vhat: lists of R arrays [N][H][d], the prefix's dequantised loop-r
    cache; tail_k, tail_v: lists of R arrays [T][H][d], the always-included
    columns at positions N..N+T-1 (the last is the token itself); q: list of
    R arrays [H][d].  Every step is a call of the pinned C oracle on an
    (N + T)-position problem with one query row at position N + T - 1.
    Returns per-loop dicts as ``run_decode``."""
    override = override or {}
    H, d, R = (sched[x] for x in ("H", "d", "R"))
    N = np.asarray(khat[0]).shape[0]
    T = np.asarray(tail_k[0]).shape[0]
    sm = F32(1.0 / np.sqrt(d))
    rows = np.array([N + T - 1], np.int32)
    S, k_cur, cstat = None, N, None
    prev = None   # (Q, K, V, lse, mu, ou) of the previous loop
    recs = []
    for r in range(1, R + 1):
        Q = np.zeros((N + T, H, d), F32)
        Q[N + T - 1] = np.asarray(q[r - 1], F32)
        K = np.concatenate([np.asarray(khat[r - 1], F32), np.asarray(tail_k[r - 1], F32)], axis=0)
        V = np.concatenate([np.asarray(vhat[r - 1], F32), np.asarray(tail_v[r - 1], F32)], axis=0)
        if r == 1:
            o, lse = attend(Q, K, V, rows, None, sm)
            mu = np.zeros((1, H), F32); ou = np.zeros((1, H, d), F32)
            need_c = R > 1 and sched["kcols"][1] < N
            c = column_stats(Q, K, rows, None, lse, sm)[:, :N] if need_c else None
            S_new, k_new = None, N
        else:
            k_r = sched["kcols"][r - 1]
            if k_cur <= k_r:
                S_new, k_new, changed = S, k_cur, False
            else:
                S_new = select_columns(override.get(("cstat", r), cstat), S, k_r, sched["n_sink"])
                k_new, changed = k_r, True
            Qp, Kp, Vp, lse_p, mu_p, ou_p = prev
            if changed:
                mu, ou = unselected_cache(Qp, Kp, Vp, rows,
                                          None if S is None else _with_tail(S, N, T),
                                          _with_tail(S_new, N, T), lse_p, sm,
                                          None if S is None else mu_p,
                                          None if S is None else ou_p)
            else:
                mu, ou = mu_p, ou_p
            ext = None if S_new is None else _with_tail(S_new, N, T)
            o, lse = attend(Q, K, V, rows, ext, sm, mu, ou)
            need_c = r < R and sched["kcols"][r] < k_new
            c = column_stats(Q, K, rows, ext, lse, sm, mu)[:, :k_new] if need_c else None
        recs.append(dict(r=r, sel=S_new, k=k_new, out=o[0], lse=lse[0], mass_u=mu[0],
                         out_u=ou[0], cstat=c))
        prev = (Q, K, V, lse, mu, ou)
        S, k_cur, cstat = S_new, k_new, c
    return recs


def run_decode(cache, q, k_self, v_self, sched, override=None):
    """Loops 1..R of one sequence's new token.

    cache: output of ``build_cache``; q, k_self, v_self: lists of R fp32
    arrays [H][d].  override: {('cstat', r): [H][k_{r-1}]} -- the GPU's own
    statistic for the column selection made at loop r.
    Returns per-loop dicts: sel [H][k] prefix columns (None when dense), k,
    out [H][d], lse [H], mass_u [H], out_u [H][d], cstat [H][k] or None."""
    R = sched["R"]
    return decode_token([cache[r]["khat"] for r in range(R)], [cache[r]["vhat"] for r in range(R)],
                        q, [np.asarray(k_self[r], F32)[None] for r in range(R)],
                        [np.asarray(v_self[r], F32)[None] for r in range(R)], sched, override)


def append_token(k_loops, v_loops, sched):
    """Generation-time growth of the cache (Sec. 4.3, App. E): a generated
    token, computed in every loop, stored as a base level (its loop-1 K/V)
    plus one residual level per later loop against its dequantised value.
    k_loops, v_loops: lists of R arrays [H][d].  Returns per level the codes
    and scales ([1][H][d], [1][H][d/g]) and the token's dequantised loop-r
    K/V ([H][d]) for r = 1..R."""
    g = sched["g"]
    out = []
    kh = vh = None
    for r in range(1, sched["R"] + 1):
        bits = sched["bits"][r - 1]
        kc, ks, _, kh = quantize_rows(np.asarray(k_loops[r - 1], F32)[None], kh, g, bits)
        vc, vs, _, vh = quantize_rows(np.asarray(v_loops[r - 1], F32)[None], vh, g, bits)
        out.append(dict(k_codes=kc, k_scale=ks, v_codes=vc, v_scale=vs, khat=kh[0], vhat=vh[0]))
    return out


def append_block(k_block, v_block, sched):
    """Generation-time growth under the paper's quantiser (App. E): its keys
    are quantised per channel over g consecutive rows, so generated tokens
    join the cache g at a time, as one new key group per level (the prompt's
    last, possibly partial, group is left as it is).  Every generated token
    is computed in all loops, so each level gains the same g rows: the base
    level quantises their loop-1 K/V, level r - 1 the residual of their
    loop-r K/V against the dequantised chain below it.
    k_block, v_block: lists of g per-token lists of R arrays [H][d].  Returns
    per level codes ([g][H][d]), scales / zeros (keys [1][H][d], values
    [g][H][d/g]) and the block's dequantised loop-r K/V [g][H][d]."""
    g = sched["g"]
    assert len(k_block) == g and len(v_block) == g
    out = []
    kh = vh = None
    for r in range(1, sched["R"] + 1):
        bits = sched["bits"][r - 1]
        kx = np.stack([np.asarray(t[r - 1], F32) for t in k_block])
        vx = np.stack([np.asarray(t[r - 1], F32) for t in v_block])
        kc, ks, kz, kh = quantize_rows_asym(kx, kh, g, bits, True)
        vc, vs, vz, vh = quantize_rows_asym(vx, vh, g, bits, False)
        out.append(dict(k_codes=kc, k_scale=ks, k_zero=kz, v_codes=vc, v_scale=vs, v_zero=vz,
                        khat=kh, vhat=vh))
    return out


def run_generation(cache, gen_q, gen_k, gen_v, sched, window=64, override=None):
    """Generation after a prompt whose cache ``build_cache`` made.

    gen_q/k/v[t]: lists of R arrays [H][d], the t-th generated token's
    per-loop query / key / value.  The most recent ``window`` generated tokens
    stay unquantised (App. E keeps the most recent 64 tokens in BF16) and
    leave the window in blocks of F tokens, oldest first: F = 1 under the
    absmax scheme (per-token groups; ``append_token``), F = g under the
    paper's quantiser (a key group is g rows; ``append_block``).  Before token
    t is decoded, while more than window + F - 1 earlier generated tokens are
    unquantised, the oldest F are appended to the cache; token t then attends
    to the quantised cache plus the generated tokens not yet appended and
    itself (between window and window + F - 1 earlier ones once appends have
    begun).  override: {t: {('cstat', r): ...}} per token.
    Returns per token a dict: recs (per-loop records of ``decode_token``), N
    (cached positions), T (window columns incl. the token), appended (None or
    the list of ``append_token`` / ``append_block`` records made before it)."""
    override = override or {}
    R = sched["R"]
    asym = sched.get("quant", "absmax") == "asym"
    F = sched["g"] if asym else 1
    khat = [np.asarray(cache[r]["khat"], F32) for r in range(R)]
    vhat = [np.asarray(cache[r]["vhat"], F32) for r in range(R)]
    out = []
    f = 0                                   # generated tokens appended so far
    for t in range(len(gen_q)):
        appended = None
        while t - f >= window + F:
            if asym:
                rec = append_block(gen_k[f:f + F], gen_v[f:f + F], sched)
                new_k = [rec[r]["khat"] for r in range(R)]
                new_v = [rec[r]["vhat"] for r in range(R)]
            else:
                rec = append_token(gen_k[f], gen_v[f], sched)
                new_k = [rec[r]["khat"][None] for r in range(R)]
                new_v = [rec[r]["vhat"][None] for r in range(R)]
            for r in range(R):
                khat[r] = np.concatenate([khat[r], new_k[r]], axis=0)
                vhat[r] = np.concatenate([vhat[r], new_v[r]], axis=0)
            appended = (appended or []) + [rec]
            f += F
        tk = [np.stack([np.asarray(gen_k[u][r], F32) for u in range(f, t + 1)]) for r in range(R)]
        tv = [np.stack([np.asarray(gen_v[u][r], F32) for u in range(f, t + 1)]) for r in range(R)]
        recs = decode_token(khat, vhat, gen_q[t], tk, tv, sched, override.get(t))
        out.append(dict(recs=recs, N=khat[0].shape[0], T=t + 1 - f, appended=appended))
    return out
