"""Pins of the looped-block oracle (no GPU): RMSNorm, RoPE and SiLU against
closed forms and invariants, and the whole dense block (rho = 1, all
columns, unquantised residuals) against a torch fp64 reference built from
library routines (rms_norm, scaled_dot_product_attention, silu)."""
import numpy as np
import torch

from oracle import block as ob
from sparse_attention_kv_amd import synth


def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0], [-2.0, 2.0]], np.float32)
    w = np.array([1.0, 2.0], np.float32)
    got = ob.rmsnorm(x, w, 0.0)
    want = np.array([[3 / np.sqrt(12.5), 2 * 4 / np.sqrt(12.5)], [-1.0, 2.0]])
    np.testing.assert_allclose(got, want, rtol=1e-6)
    rng = np.random.default_rng(0)
    y = rng.standard_normal((5, 64)).astype(np.float32)
    np.testing.assert_allclose(ob.rmsnorm(7.5 * y, np.ones(64), 0.0), ob.rmsnorm(y, np.ones(64), 0.0), rtol=1e-5)


def test_rope_invariants():
    """Identity at position 0, pairwise norms kept, and q.k depends only on
    the position difference (catches a swapped sin sign or wrong frequency
    index)."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, 64)).astype(np.float32)
    k = rng.standard_normal((1, 2, 64)).astype(np.float32)
    np.testing.assert_array_equal(ob.rope(q, [0], 1e4), q)
    r = ob.rope(q, [37], 1e4)
    n0 = q[..., :32] ** 2 + q[..., 32:] ** 2
    n1 = r[..., :32] ** 2 + r[..., 32:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-5)
    for p, pk, s in [(10, 3, 100), (500, 499, 7)]:
        a = np.sum(ob.rope(q, [p], 1e4) * ob.rope(k, [pk], 1e4), axis=-1)
        b = np.sum(ob.rope(q, [p + s], 1e4) * ob.rope(k, [pk + s], 1e4), axis=-1)
        np.testing.assert_allclose(a, b, rtol=2e-4, atol=2e-4)
    # one-hot frequency check: x = e_i rotates by pos * theta^(-2i/d)
    e = np.zeros((1, 1, 8), np.float32); e[0, 0, 1] = 1.0
    out = ob.rope(e, [3], 100.0)
    ang = 3 * 100.0 ** (-2 / 8)
    np.testing.assert_allclose(out[0, 0, [1, 5]], [np.cos(ang), np.sin(ang)], rtol=1e-5)


def test_bf16_rounding():
    # 1 + 2^-8 is a tie (to even: 1.0); one fp32 ulp above it rounds up
    x = np.array([1.0, 1.00390625, 1.01171875, -3.0078125, 0.0], np.float32)
    x[4] = np.array([0x3F808001], np.uint32).view(np.float32)[0]
    np.testing.assert_array_equal(ob.bf16(x), [1.0, 1.0, 1.015625, -3.0, 1.0078125])


def test_silu():
    np.testing.assert_allclose(ob.silu(np.array([0.0, 20.0, -20.0])), [0.0, 20.0, -20 / (1 + np.exp(20))],
                               rtol=1e-6, atol=1e-12)


def _torch_block(h, weights, R, H, d, theta, eps):
    """Dense reference: R loops of the layers on every token, fp64 torch."""
    x = torch.from_numpy(np.asarray(h, np.float64))
    N, D = x.shape
    pos = torch.arange(N, dtype=torch.float64)
    inv = theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = pos[:, None] * inv[None, :]
    cs, sn = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rot(t):
        t1, t2 = t[..., : d // 2], t[..., d // 2:]
        return torch.cat([t1 * cs - t2 * sn, t2 * cs + t1 * sn], dim=-1)

    W = [{k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in lw.items()} for lw in weights]
    for _ in range(R):
        for w in W:
            a = torch.nn.functional.rms_norm(x, (D,), w["norm1"], eps)
            qkv = a @ w["w_qkv"].T
            q = rot(qkv[:, :D].reshape(N, H, d)).permute(1, 0, 2)[None]
            k = rot(qkv[:, D:2 * D].reshape(N, H, d)).permute(1, 0, 2)[None]
            v = qkv[:, 2 * D:].reshape(N, H, d).permute(1, 0, 2)[None]
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
            x = x + o[0].permute(1, 0, 2).reshape(N, D) @ w["w_o"].T
            b = torch.nn.functional.rms_norm(x, (D,), w["norm2"], eps)
            gu = b @ w["w_gu"].T
            x = x + (torch.nn.functional.silu(gu[:, 0::2]) * gu[:, 1::2]) @ w["w_down"].T
    return x.numpy()


def test_dense_block_matches_torch():
    """rho = 1, k = N, unquantised residuals (raw base too): the oracle's
    looped block equals the dense reference loop after loop."""
    w = synth.WORKLOADS["block8k"].scaled(N=48, H=2, d=64, R=2, rho=[1.0, 1.0], kcols=[48, 48],
                                          bits=[32, 32])
    w.extra = dict(w.extra, layers=2, ffn=96, wstd=0.05)
    inp = synth.generate(w)
    layers = [{k: synth.bf16_bits_to_f32(v) for k, v in lw.items()} for lw in inp["layers"]]
    res = ob.run_block(inp["h1"], layers, w.sched(), theta=1e4, eps=1e-6)
    for r in range(1, 3):
        ref = _torch_block(inp["h1"], layers, r, 2, 64, 1e4, 1e-6)
        np.testing.assert_allclose(res[r - 1]["h"], ref, rtol=0, atol=5e-4 * np.abs(ref).max())
    # inactive rows never move: a sparse loop keeps them bit-identical
    w2 = synth.WORKLOADS["block8k"].scaled(N=48, H=2, d=64, R=2, rho=[1.0, 0.25], kcols=[48, 16],
                                           bits=[8, 4])
    w2.extra = dict(w2.extra, layers=2, ffn=96, wstd=0.05)
    res2 = ob.run_block(inp["h1"], layers, w2.sched())
    inactive = np.setdiff1d(np.arange(48), res2[1]["active"])
    np.testing.assert_array_equal(res2[1]["h"][inactive], res2[0]["h"][inactive])
