"""Oracle of the token-sparse looped block: R loops of an n_layers pre-norm
Transformer block whose layers run only on each loop's active tokens.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

FlashLoop paper, Sec. 4.1 (the looped block computes only the selected active
tokens; inactive tokens keep their states and reuse their K/V), Sec. 4.2-4.3
(per-layer sparse attention and residual KV cache, as in ``loop.py``), App. E
(keys are quantised after RoPE).  The layer is the usual pre-norm block the
workload names (RMSNorm, RoPE, SwiGLU MLP):

    a = RMSNorm(h) * norm1,  [q k v] = a W_qkv^T,  q, k <- RoPE at the token
    position,  h += Attention(q, K, V) W_o^T,
    b = RMSNorm(h) * norm2,  h += (silu(b W_g^T) * (b W_u^T)) W_down^T,
    RMSNorm(x) = x / sqrt(mean(x^2) + eps),  silu(x) = x / (1 + exp(-x)),
    RoPE (rotate-half): for i < d/2, angle = pos * theta^(-2i/d),
        (x_i, x_{i+d/2}) -> (x_i cos - x_{i+d/2} sin, x_{i+d/2} cos + x_i sin).

Everything is fp32 numpy; the projections use numpy's matmul.  The residual
stream h is fp32.  Attention, quantisation and selection call the C oracle.

With bf16_acts (the block workload is a bf16 model) the activations take
bf16 values where a bf16 model stores them: the normed inputs of the
projections, the projected q/k/v (q and k after RoPE), the attention output
entering W_o and the SwiGLU output entering W_down (round to nearest even);
products accumulate in fp32 and the residual stream stays fp32.  Both sides
then quantise the same K/V values, so codes are decided identically.
"""
from __future__ import annotations

import numpy as np

from . import (active_count, attend, column_stats, delta_norm, quantize_rows,
               quantize_rows_asym, select_columns, top_select, unselected_cache)

F32 = np.float32


def rmsnorm(x, w, eps):
    x = np.asarray(x, F32)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    return (x / np.sqrt(ms + F32(eps))) * np.asarray(w, F32)


def rope(x, pos, theta):
    """x [n][H][d] fp32, pos [n] token positions."""
    x = np.asarray(x, F32)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=F32)
    inv = np.power(F32(theta), -(F32(2) * i) / F32(d)).astype(F32)
    ang = (np.asarray(pos, F32)[:, None] * inv[None, :]).astype(F32)
    cs = np.cos(ang)[:, None, :].astype(F32)
    sn = np.sin(ang)[:, None, :].astype(F32)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * cs - x2 * sn, x2 * cs + x1 * sn], axis=-1).astype(F32)


def bf16(x):
    """Round fp32 values to bf16 (nearest, ties to even), returned as fp32."""
    u = np.ascontiguousarray(x, F32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(F32)


def silu(x):
    x = np.asarray(x, F32)
    return x / (F32(1) + np.exp(-x))


def _level(xnew, xprev, g, bits, asym=False, per_channel=False):
    if asym:
        codes, scales, zeros, xhat = quantize_rows_asym(xnew, xprev, g, bits, per_channel)
        return dict(codes=codes, scales=scales, zeros=zeros, raw=None), xhat
    codes, scales, raw, xhat = quantize_rows(xnew, xprev, g, bits)
    return dict(codes=codes, scales=scales, raw=raw), xhat


def unpack_codes(packed, bits, d, unsigned=False):
    """Codes from their packed bytes ([..][d*bits/8] -> [..][d]): two's
    complement, or unsigned (the asymmetric quantiser's codes)."""
    b = np.asarray(packed, np.uint8)
    per = 8 // bits
    out = np.empty(b.shape[:-1] + (b.shape[-1] * per,), np.int16)
    for i in range(per):
        v = ((b >> (bits * i)) & ((1 << bits) - 1)).astype(np.int16)
        out[..., i::per] = v if unsigned else np.where(v >= (1 << (bits - 1)), v - (1 << bits), v)
    return out[..., :d]


def dequant_rows_asym(codes_packed, scales, zeros, bits, g, xhat_prev, per_channel):
    """Rows of one level of the asymmetric quantiser from stored codes:
    code*s + z per element (keys: s, z per (row group of g, channel); values:
    per (row, channel group of g)), plus the previous level's value."""
    n = np.asarray(codes_packed).shape[0]
    d = np.asarray(codes_packed).shape[-1] * 8 // bits
    c = unpack_codes(codes_packed, bits, d, unsigned=True).astype(F32)
    if per_channel:
        sc = np.repeat(np.asarray(scales, F32), g, axis=0)[:n]
        zc = np.repeat(np.asarray(zeros, F32), g, axis=0)[:n]
    else:
        sc = np.repeat(np.asarray(scales, F32), g, axis=-1)
        zc = np.repeat(np.asarray(zeros, F32), g, axis=-1)
    deq = ((c * sc).astype(F32) + zc).astype(F32)
    return deq if xhat_prev is None else (np.asarray(xhat_prev, F32) + deq).astype(F32)


def run_block(h1, weights, sched, theta=10000.0, eps=1e-6, override=None, bf16_acts=False):
    """h1: [N][D] input hidden states; weights: list per layer of dicts of fp32
    arrays w_qkv [3D][D], w_o [D][D], w_gu [2F][D] (rows 2j gate, 2j+1 up),
    w_down [D][F], norm1 [D], norm2 [D].  sched as in ``loop.run_prefill``.
    override: {('stat', r): array, ('cstat', r, layer): array} -- the GPU's own
    statistics for the selections of loop r; ('kvin', r, layer): dict(k=, v=)
    of [n_r][H][d] fp32 -- another implementation's keys (after RoPE) and
    values of the active rows, which the oracle's quantiser then quantises in
    place of the oracle's own projections (these are still computed and
    returned as k_in / v_in for comparison).  The quantiser itself, the cache
    it builds and everything downstream stay the oracle's.
    Returns per-loop records."""
    override = override or {}
    rd = bf16 if bf16_acts else (lambda z: np.asarray(z, F32))
    N, H, d, g, R = (sched[x] for x in ("N", "H", "d", "g", "R"))
    D = H * d
    sm = F32(1.0 / np.sqrt(d))
    n_sink = sched["n_sink"]
    L = len(weights)
    h = np.array(h1, F32, copy=True)
    h_entry = h.copy()
    st = [dict(khat=None, vhat=None, q=np.zeros((N, H, d), F32), lse=np.zeros((N, H), F32),
               mu=np.zeros((N, H), F32), ou=np.zeros((N, H, d), F32), S=None, k=N, cstat=None)
          for _ in range(L)]
    A = np.arange(N, dtype=np.int32)
    rel = sched.get("token_stat", "abs") == "rel"
    vw = sched.get("col_stat", "mass") == "vnorm"
    asym = sched.get("quant", "absmax") == "asym"
    out = []
    for r in range(1, R + 1):
        rec = dict(r=r)
        if r > 1:
            stat = delta_norm(h, h_entry, A, relative=rel)
            n_r = active_count(sched["rho"][r - 1], N, len(A))
            A = top_select(override.get(("stat", r), stat), n_r, A)
            rec["stat"] = stat
        rec["active"] = A
        h_entry = h.copy()
        rec["layers"] = []
        for l, w in enumerate(weights):
            s = st[l]
            a = rd(rmsnorm(h[A], w["norm1"], eps))
            qkv = rd(a @ np.asarray(w["w_qkv"], F32).T)
            q = rd(rope(qkv[:, :D].reshape(-1, H, d), A, theta))
            k = rd(rope(qkv[:, D:2 * D].reshape(-1, H, d), A, theta))
            v = np.ascontiguousarray(qkv[:, 2 * D:].reshape(-1, H, d))
            bits = sched["bits"][r - 1]
            kp = None if r == 1 else s["khat"][A]
            vp = None if r == 1 else s["vhat"][A]
            ext = override.get(("kvin", r, l))
            kq = k if ext is None else np.asarray(ext["k"], F32).reshape(k.shape)
            vq = v if ext is None else np.asarray(ext["v"], F32).reshape(v.shape)
            lk, krows = _level(kq, kp, g, bits, asym, True)
            lv, vrows = _level(vq, vp, g, bits, asym, False)
            if r == 1:
                khat, vhat = krows, vrows
            else:
                khat = s["khat"].copy(); khat[A] = krows
                vhat = s["vhat"].copy(); vhat[A] = vrows
            qd = s["q"].copy(); qd[A] = q
            lrec = dict(level_k=lk, level_v=lv, k_in=k, v_in=v)
            if r == 1:
                o, lse = attend(qd, khat, vhat, None, None, sm)
                mu = np.zeros((N, H), F32); ou = np.zeros((N, H, d), F32)
                S_new, k_new = None, N
                need_c = R > 1 and sched["kcols"][1] < N
                c = column_stats(qd, khat, None, None, lse, sm,
                                 vhat=vhat if vw else None) if need_c else None
            else:
                k_r = sched["kcols"][r - 1]
                if s["k"] <= k_r:
                    S_new, k_new, changed = s["S"], s["k"], False
                else:
                    cs = override.get(("cstat", r, l), s["cstat"])
                    S_new = select_columns(cs, s["S"], k_r, n_sink)
                    k_new, changed = k_r, True
                if changed:
                    mu, ou = unselected_cache(s["q"], s["khat"], s["vhat"], A, s["S"], S_new,
                                              s["lse"][A], sm,
                                              None if s["S"] is None else s["mu"][A],
                                              None if s["S"] is None else s["ou"][A])
                else:
                    mu, ou = s["mu"][A].copy(), s["ou"][A].copy()
                o, lse = attend(qd, khat, vhat, A, S_new, sm, mu, ou)
                need_c = r < R and sched["kcols"][r] < k_new
                c = column_stats(qd, khat, A, S_new, lse, sm, mu,
                                 vhat=vhat if vw else None) if need_c else None
            lrec.update(sel=S_new, k=k_new, out=o, lse=lse, mass_u=mu, cstat=c)
            rec["layers"].append(lrec)
            # carry the layer's state
            s["q"] = qd
            s["khat"], s["vhat"] = khat, vhat
            s["lse"] = s["lse"].copy(); s["lse"][A] = lse
            s["mu"] = s["mu"].copy(); s["mu"][A] = mu
            s["ou"] = s["ou"].copy(); s["ou"][A] = ou
            s["S"], s["k"], s["cstat"] = S_new, k_new, c
            # rest of the layer on the active rows
            h[A] += (rd(o.reshape(-1, D)) @ np.asarray(w["w_o"], F32).T).astype(F32)
            b = rd(rmsnorm(h[A], w["norm2"], eps))
            gu = (b @ np.asarray(w["w_gu"], F32).T).astype(F32)
            mlp = rd(silu(gu[:, 0::2]) * gu[:, 1::2])
            h[A] += (mlp @ np.asarray(w["w_down"], F32).T).astype(F32)
        rec["h"] = h.copy()
        out.append(rec)
    return out
