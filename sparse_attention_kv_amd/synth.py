"""Seeded synthetic inputs for the lazy-update loop attention step.

This module only draws random inputs and describes workload shapes and
schedules; it holds none of the method's arithmetic.  Both the GPU library's
tests/benchmark and the CPU oracle consume the same arrays from here.

Random numbers: numpy PCG64 with a fixed seed per workload and a fixed draw
order.  Values are drawn in fp32; bf16 workloads round each per-loop tensor to
bf16 (round to nearest even), and both sides read the same bf16 bytes (the
oracle reads their exact fp32 expansion).

Inputs per loop r (0-based list index r-1): the hidden state entering the loop
h_r [N][D], and the loop's query/key/value rows q_r, k_r, v_r [N][H][d].  In
this attention-only harness the loop's projections are given; the method
decides which rows of them it uses.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np


# --------------------------------------------------------------------------
# bf16 helpers (bit manipulation of IEEE fp32; round to nearest even)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs only: u + 0x7fff + lsb cannot wrap below the NaN range
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 values of a stored tensor (bf16 bits or fp32)."""
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


# --------------------------------------------------------------------------
# Workload table

@dataclass
class Workload:
    name: str
    N: int
    H: int
    d: int
    R: int
    g: int
    n_sink: int
    rho: list            # per loop, fraction of N kept active (rho[0] == 1)
    kcols: list          # per loop, column budget (kcols[0] == N: dense first loop)
    bits: list           # per loop: bits[0] base (8), later residual bits (4/2)
    dtype: str           # "f32" or "bf16"
    seed: int
    kind: str = "prefill"   # "tiny", "prefill", "decode", "block"
    sigma_mu: tuple = (-2.0, -0.5)   # log sigma mean = a + b*r
    sigma_sd: float = 1.0
    boost_frac: float = 0.03
    extra: dict = field(default_factory=dict)

    @property
    def D(self) -> int:
        return self.H * self.d

    def sched(self) -> dict:
        return dict(N=self.N, H=self.H, d=self.d, g=self.g, R=self.R, n_sink=self.n_sink,
                    rho=list(self.rho), kcols=list(self.kcols), bits=list(self.bits))

    def scaled(self, **kw) -> "Workload":
        """Same recipe at other sizes; column budgets scale with N unless given."""
        w = dataclasses.replace(self, **kw)
        if "N" in kw and "kcols" not in kw:
            ratio = kw["N"] / self.N
            kc = [kw["N"]] + [max(w.n_sink + 1, int(round(c * ratio))) for c in self.kcols[1:]]
            w = dataclasses.replace(w, kcols=kc)
        return w


def depth_schedule(R: int, N: int):
    """Per-loop budgets of the deep recipe: kept fraction 0.5 at loop 2,
    shrinking by 0.9 a loop down to 0.02; columns 2048 shrinking by 0.9 a loop
    down to 256; int8 base, int4 residuals at loops 2-8, int2 after."""
    rho = [1.0] + [round(max(0.02, 0.5 * 0.9 ** (r - 2)), 4) for r in range(2, R + 1)]
    kc = [N] + [max(256, int(2048 * 0.9 ** (r - 2))) for r in range(2, R + 1)]
    bits = [8] + [4 if r <= 8 else 2 for r in range(2, R + 1)]
    return rho, kc, bits


_DEPTH_RHO, _DEPTH_K, _DEPTH_BITS = depth_schedule(32, 8192)

WORKLOADS = {
    # 1 head x 64, seq 256, R=2, fp32; rho 0.25, 64 columns incl. 4 sinks;
    # int8 base / int4 residual, group 32.
    "tiny": Workload("tiny", N=256, H=1, d=64, R=2, g=32, n_sink=4, rho=[1.0, 0.25],
                     kcols=[256, 64], bits=[8, 4], dtype="f32", seed=0, kind="tiny"),
    # one looped attention layer, 16 x 128, seq 4096, R=4, bf16; rho 0.2, k 512,
    # int8 base + int4 residuals, group 64.
    "layer4k": Workload("layer4k", N=4096, H=16, d=128, R=4, g=64, n_sink=4,
                        rho=[1.0, 0.2, 0.2, 0.2], kcols=[4096, 512, 512, 512],
                        bits=[8, 4, 4, 4], dtype="bf16", seed=1, sigma_sd=1.0),
    # long-context prefill, 16 x 128, seq 32768, R=4, bf16; active fractions
    # 1/.4/.2/.1; 2048 columns incl. 4 sinks; int4 at loop 2, int2 at 3-4.
    "prefill32k": Workload("prefill32k", N=32768, H=16, d=128, R=4, g=64, n_sink=4,
                           rho=[1.0, 0.4, 0.2, 0.1], kcols=[32768, 2048, 2048, 2048],
                           bits=[8, 4, 2, 2], dtype="bf16", seed=2, sigma_sd=1.5),
    # full looped block: 24 layers of shared random-init weights, hidden 2048
    # (16 x 128), SwiGLU 5632, RMSNorm (eps 1e-6), RoPE (theta 1e4), R=4,
    # seq 8192; fractions 1/.4/.2/.1, 1024 columns incl. 4 sinks, int8 base,
    # int4 at loop 2 and int2 at loops 3-4, group 64.
    # batched decode: 64 sequences x 8192 cached tokens (each cache built as
    # the prefill recipe at N=8192, fractions 1/.4/.2/.1, int8 base + int4
    # residuals at every loop), one new query per sequence per loop, R=4,
    # 16 x 128; loop 1 dense over the prefix, loops 2-4 on 256 columns
    # (4 sinks), plus the token's own column.
    # deep looping: 32 loops at seq 8192 (16 x 128, bf16), per-loop kept
    # fractions and column budgets shrinking with depth (depth_schedule);
    # per-token loop updates decay slowly, log sigma = -2.4 - 0.09 r.
    "depth32x8k": Workload("depth32x8k", N=8192, H=16, d=128, R=32, g=64, n_sink=4,
                           rho=_DEPTH_RHO, kcols=_DEPTH_K, bits=_DEPTH_BITS, dtype="bf16",
                           seed=5, sigma_mu=(-2.4, -0.09), sigma_sd=1.0),
    "decode64x8k": Workload("decode64x8k", N=8192, H=16, d=128, R=4, g=64, n_sink=4,
                            rho=[1.0, 0.4, 0.2, 0.1], kcols=[8192, 256, 256, 256],
                            bits=[8, 4, 4, 4], dtype="bf16", seed=3, kind="decode",
                            sigma_sd=1.5, extra=dict(B=64)),
    "block8k": Workload("block8k", N=8192, H=16, d=128, R=4, g=64, n_sink=4,
                        rho=[1.0, 0.4, 0.2, 0.1], kcols=[8192, 1024, 1024, 1024],
                        bits=[8, 4, 2, 2], dtype="bf16", seed=4, kind="block",
                        extra=dict(layers=24, ffn=5632, theta=10000.0, eps=1e-6, wstd=0.02)),
}


# --------------------------------------------------------------------------
# Generators

def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def gen_tiny(w: Workload) -> dict:
    """Tiny case: h_1, K_1, V_1 ~ N(0,1); q_r is h_r (H*d == D); per-token
    loop-2 delta scale sigma_i = exp(N(-3,1)), 25% of tokens scaled x20."""
    rng = _rng(w.seed)
    N, D = w.N, w.D
    h1 = rng.standard_normal((N, D), dtype=np.float32)
    k1 = rng.standard_normal((N, D), dtype=np.float32)
    v1 = rng.standard_normal((N, D), dtype=np.float32)
    sig = np.exp(rng.normal(-3.0, 1.0, N)).astype(np.float32)
    boost = rng.choice(N, size=N // 4, replace=False)
    sig[boost] *= np.float32(20.0)
    hs, ks, vs = [h1], [k1], [v1]
    for _ in range(1, w.R):
        hs.append(hs[-1] + sig[:, None] * rng.standard_normal((N, D), dtype=np.float32))
        ks.append(ks[-1] + sig[:, None] * rng.standard_normal((N, D), dtype=np.float32))
        vs.append(vs[-1] + sig[:, None] * rng.standard_normal((N, D), dtype=np.float32))
    shp = (N, w.H, w.d)
    return dict(h=hs, q=[x.reshape(shp).copy() for x in hs], k=[x.reshape(shp) for x in ks],
                v=[x.reshape(shp) for x in vs], dtype="f32")


def gen_prefill(w: Workload) -> dict:
    """Ouro-class layer: per-head mean query direction m_h ~ N(0, I_d);
    q_1 = m_h + N(0,I); K_1, V_1 ~ N(0,I); h_1 ~ N(0, I_D).  Per head a
    fraction boost_frac of columns (drawn from positions >= 4) get
    K_1 += 3 m_h/|m_h| (about +3 logits).  Loop r >= 2: per-token
    sigma = exp(N(a + b*r, sigma_sd)); h, q, K, V each get + sigma * N(0, I),
    accumulated in fp32 and rounded to bf16 per loop."""
    rng = _rng(w.seed)
    N, H, d, D = w.N, w.H, w.d, w.D
    m = rng.standard_normal((H, d), dtype=np.float32)
    q = m[None] + rng.standard_normal((N, H, d), dtype=np.float32)
    k = rng.standard_normal((N, H, d), dtype=np.float32)
    v = rng.standard_normal((N, H, d), dtype=np.float32)
    h = rng.standard_normal((N, D), dtype=np.float32)
    nb = int(round(w.boost_frac * N))
    unit = m / np.linalg.norm(m, axis=1, keepdims=True)
    for hh in range(H):
        cols = rng.choice(np.arange(4, N), size=nb, replace=False)
        k[cols, hh, :] += np.float32(3.0) * unit[hh]
    cast = f32_to_bf16_bits if w.dtype == "bf16" else (lambda x: x.copy())
    hs, qs, ks, vs = [cast(h)], [cast(q)], [cast(k)], [cast(v)]
    a, b = w.sigma_mu
    for r in range(2, w.R + 1):
        sig = np.exp(rng.normal(a + b * r, w.sigma_sd, N)).astype(np.float32)
        h += sig[:, None] * rng.standard_normal((N, D), dtype=np.float32)
        q += sig[:, None, None] * rng.standard_normal((N, H, d), dtype=np.float32)
        k += sig[:, None, None] * rng.standard_normal((N, H, d), dtype=np.float32)
        v += sig[:, None, None] * rng.standard_normal((N, H, d), dtype=np.float32)
        hs.append(cast(h)); qs.append(cast(q)); ks.append(cast(k)); vs.append(cast(v))
    return dict(h=hs, q=qs, k=ks, v=vs, dtype=w.dtype)


def gen_block(w: Workload) -> dict:
    """Looped block: embeddings h_1 ~ N(0,1) [N][D]; per layer weights
    ~ N(0, wstd^2), output-major: w_qkv [3D][D], w_o [D][D], w_gu [2F][D]
    (row 2j gate, row 2j+1 up of hidden unit j), w_down [D][F]; RMSNorm
    weights 1.  All stored as bf16 (round to nearest even)."""
    rng = _rng(w.seed)
    N, D = w.N, w.D
    F, L, sd = w.extra["ffn"], w.extra["layers"], np.float32(w.extra["wstd"])
    h1 = rng.standard_normal((N, D), dtype=np.float32)
    layers = []
    for _ in range(L):
        lw = {}
        for name, shape in (("w_qkv", (3 * D, D)), ("w_o", (D, D)), ("w_gu", (2 * F, D)),
                            ("w_down", (D, F))):
            lw[name] = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * sd)
        lw["norm1"] = f32_to_bf16_bits(np.ones(D, np.float32))
        lw["norm2"] = f32_to_bf16_bits(np.ones(D, np.float32))
        layers.append(lw)
    return dict(h1=h1, layers=layers, dtype="bf16")


def decode_seeds(w: Workload):
    """Independent seed sequences of the decode batch's sequences."""
    return np.random.SeedSequence(w.seed).spawn(w.extra["B"])


def gen_decode_seq(w: Workload, b: int, n_gen: int = 0) -> dict:
    """Sequence b of the decode batch.

    Prefix of N cached tokens, drawn with the prefill recipe: per-head mean
    query direction m_h ~ N(0, I_d); K_1, V_1 ~ N(0, I) with boost_frac of
    the columns (positions >= 4) given K_1 += 3 m_h/|m_h|; loop r >= 2 moves
    every token by sigma_r(i) * N(0, I) with sigma_r(i) = exp(N(a + b*r,
    sigma_sd)).  The prefix's hidden states only enter through the selection
    statistic ||h_r(i) - h_{r-1}(i)||_2, which under this recipe is
    sigma_r(i) * chi_D (D = H*d), so it is drawn directly as stat[r-1] [N]
    (None at r = 1).  K and V are given for every position at every loop
    (the method decides which rows it stores).

    The new token: q_1 = m_h + N(0, I), k_1, v_1 ~ N(0, I) [H][d]; loop
    r >= 2 adds s_r * N(0, I) to each, s_r = exp(N(a + b*r, sigma_sd)).
    All K/V/q tensors are bf16 bits.

    n_gen > 0 also draws that many generated tokens after the above (their
    draws come last, so the rest does not change): each like the new token,
    q = m_h + N(0, I), k, v ~ N(0, I), loop r >= 2 adding s_r * N(0, I) with
    its own s_r; returned as gen_q / gen_k / gen_v [t][r] of [H][d]."""
    rng = np.random.Generator(np.random.PCG64(decode_seeds(w)[b]))
    N, H, d, D = w.N, w.H, w.d, w.D
    m = rng.standard_normal((H, d), dtype=np.float32)
    k = rng.standard_normal((N, H, d), dtype=np.float32)
    v = rng.standard_normal((N, H, d), dtype=np.float32)
    nb = int(round(w.boost_frac * N))
    unit = m / np.linalg.norm(m, axis=1, keepdims=True)
    for hh in range(H):
        cols = rng.choice(np.arange(4, N), size=nb, replace=False)
        k[cols, hh, :] += np.float32(3.0) * unit[hh]
    qn = m + rng.standard_normal((H, d), dtype=np.float32)
    kn = rng.standard_normal((H, d), dtype=np.float32)
    vn = rng.standard_normal((H, d), dtype=np.float32)
    cast = f32_to_bf16_bits
    ks, vs, stats = [cast(k)], [cast(v)], [None]
    qs, kns, vns = [cast(qn)], [cast(kn)], [cast(vn)]
    a, bb = w.sigma_mu
    for r in range(2, w.R + 1):
        sig = np.exp(rng.normal(a + bb * r, w.sigma_sd, N)).astype(np.float32)
        stats.append((sig * np.sqrt(rng.chisquare(D, N)).astype(np.float32)).astype(np.float32))
        k += sig[:, None, None] * rng.standard_normal((N, H, d), dtype=np.float32)
        v += sig[:, None, None] * rng.standard_normal((N, H, d), dtype=np.float32)
        s1 = np.float32(np.exp(rng.normal(a + bb * r, w.sigma_sd)))
        qn = qn + s1 * rng.standard_normal((H, d), dtype=np.float32)
        kn = kn + s1 * rng.standard_normal((H, d), dtype=np.float32)
        vn = vn + s1 * rng.standard_normal((H, d), dtype=np.float32)
        ks.append(cast(k)); vs.append(cast(v))
        qs.append(cast(qn)); kns.append(cast(kn)); vns.append(cast(vn))
    out = dict(stat=stats, k=ks, v=vs, q_new=qs, k_new=kns, v_new=vns, dtype="bf16")
    if n_gen:
        gq, gk, gv = [], [], []
        for _ in range(n_gen):
            tq = m + rng.standard_normal((H, d), dtype=np.float32)
            tk = rng.standard_normal((H, d), dtype=np.float32)
            tv = rng.standard_normal((H, d), dtype=np.float32)
            lq, lk, lv = [cast(tq)], [cast(tk)], [cast(tv)]
            for r in range(2, w.R + 1):
                s1 = np.float32(np.exp(rng.normal(a + bb * r, w.sigma_sd)))
                tq = tq + s1 * rng.standard_normal((H, d), dtype=np.float32)
                tk = tk + s1 * rng.standard_normal((H, d), dtype=np.float32)
                tv = tv + s1 * rng.standard_normal((H, d), dtype=np.float32)
                lq.append(cast(tq)); lk.append(cast(tk)); lv.append(cast(tv))
            gq.append(lq); gk.append(lk); gv.append(lv)
        out.update(gen_q=gq, gen_k=gk, gen_v=gv)
    return out


def generate(w: Workload) -> dict:
    if w.kind == "decode":
        raise ValueError("decode inputs are drawn per sequence: gen_decode_seq(w, b)")
    if w.kind == "block":
        return gen_block(w)
    if w.kind == "tiny":
        return gen_tiny(w)
    if w.kind == "prefill":
        return gen_prefill(w)
    raise ValueError(f"no generator for kind {w.kind}")


def as_f32_inputs(inp: dict) -> dict:
    """The same inputs as exact fp32 arrays (what the oracle reads)."""
    dt = inp["dtype"]
    return {key: [to_f32(a, dt) for a in inp[key]] for key in ("h", "q", "k", "v")}
