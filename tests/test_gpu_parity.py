"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs.  Index sets, slot maps, codes and scales must match bit for
bit; floating outputs within rel-L2 1e-2 and max-abs 3e-2."""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_kv_amd import fl, synth

from gpu_chain import (assert_close, compare_chain, counts, run_gpu, run_oracle_lockstep,
                       to_dev)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------ selection --
@pytest.mark.parametrize("n_cand,n_sel,ties", [(5000, 1234, False), (3000, 3000, True),
                                               (1, 1, False), (4097, 1, True), (70000, 9000, True)])
def test_select_active_matches_oracle(n_cand, n_sel, ties):
    _say("select_active", n_cand, n_sel, ties)
    rng = np.random.default_rng(n_cand)
    N = n_cand + 50
    cand = np.sort(rng.choice(N, n_cand, replace=False)).astype(np.int32)
    if ties:
        key = rng.integers(0, 7, n_cand).astype(np.float32)
        key[rng.random(n_cand) < 0.3] = -0.0
    else:
        key = rng.random(n_cand).astype(np.float32)
    act = torch.empty(n_sel, dtype=torch.int32, device="cuda")
    slot = torch.empty(N, dtype=torch.int32, device="cuda")
    fl.fl_select_active(None, None, torch.from_numpy(cand).cuda(), n_sel, None, act, slot,
                        stat_in=torch.from_numpy(key).cuda(), N=N)
    torch.cuda.synchronize()
    want = oracle.top_select(key, n_sel, cand)
    np.testing.assert_array_equal(act.cpu().numpy(), want)
    s = np.full(N, -1, np.int32); s[want] = np.arange(n_sel)
    np.testing.assert_array_equal(slot.cpu().numpy(), s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_delta_norm_matches_oracle(dtype):
    _say("delta_norm", dtype)
    rng = np.random.default_rng(3)
    N, D = 3001, 2048 if dtype == "bf16" else 64
    a = rng.standard_normal((N, D)).astype(np.float32)
    b = a + (rng.standard_normal((N, D)) * np.exp(rng.normal(-3, 1, (N, 1)))).astype(np.float32)
    if dtype == "bf16":
        a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    cand = np.sort(rng.choice(N, 1500, replace=False)).astype(np.int32)
    stat = torch.empty(1500, dtype=torch.float32, device="cuda")
    act = torch.empty(300, dtype=torch.int32, device="cuda")
    fl.fl_select_active(to_dev(a, dtype), to_dev(b, dtype), torch.from_numpy(cand).cuda(), 300,
                        stat, act)
    torch.cuda.synchronize()
    g = stat.cpu().numpy()
    want = oracle.delta_norm(synth.to_f32(a, dtype), synth.to_f32(b, dtype), cand)
    np.testing.assert_allclose(g, want, rtol=1e-5)
    np.testing.assert_array_equal(act.cpu().numpy(), oracle.top_select(g, 300, cand))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_delta_norm_rel_matches_oracle(dtype):
    """Normalised token change (Sec. 4.1): ratio within 1e-5, zero previous
    states (unchanged -> 0, changed -> +inf) exact, and the selection equal
    to the oracle's top-k of the GPU's own statistic."""
    _say("delta_norm_rel", dtype)
    rng = np.random.default_rng(5)
    N, D = 2051, 2048 if dtype == "bf16" else 64
    b = (rng.standard_normal((N, D)) * np.exp(rng.normal(0, 1, (N, 1)))).astype(np.float32)
    a = b + (rng.standard_normal((N, D)) * np.exp(rng.normal(-3, 1, (N, 1)))).astype(np.float32)
    b[7] = 0; a[7] = 0            # unchanged zero state
    b[11] = 0                     # changed zero state
    if dtype == "bf16":
        a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    cand = np.sort(np.concatenate([[7, 11], 12 + rng.choice(N - 12, 1198, replace=False)])).astype(np.int32)
    stat = torch.empty(1200, dtype=torch.float32, device="cuda")
    act = torch.empty(250, dtype=torch.int32, device="cuda")
    fl.fl_select_active(to_dev(a, dtype), to_dev(b, dtype), torch.from_numpy(cand).cuda(), 250,
                        stat, act, stat_kind=fl.FL_TOKEN_STAT_REL)
    torch.cuda.synchronize()
    g = stat.cpu().numpy()
    want = oracle.delta_norm(synth.to_f32(a, dtype), synth.to_f32(b, dtype), cand, relative=True)
    assert g[0] == 0 and np.isposinf(g[1]) and want[0] == 0 and np.isposinf(want[1])
    np.testing.assert_allclose(g[2:], want[2:], rtol=1e-5)
    got_act = act.cpu().numpy()
    np.testing.assert_array_equal(got_act, oracle.top_select(g, 250, cand))
    assert 11 in got_act and 7 not in got_act


@pytest.mark.parametrize("H,n_cand,k,ident", [(3, 3000, 500, True), (16, 2048, 1024, False),
                                              (2, 100, 5, False), (4, 700, 700, False)])
def test_select_columns_matches_oracle(H, n_cand, k, ident):
    _say("select_columns", H, n_cand, k, ident)
    rng = np.random.default_rng(k)
    ns = 4
    if ident:
        cand = None
    else:
        cand = np.stack([np.sort(np.concatenate([np.arange(ns), ns + rng.choice(
            5 * n_cand, n_cand - ns, replace=False)])) for _ in range(H)]).astype(np.int32)
    cs = rng.integers(0, 9, (H, n_cand)).astype(np.float32)
    k_out = min(k, n_cand)
    sel = torch.empty((H, k_out), dtype=torch.int32, device="cuda")
    fl.fl_select_columns(torch.from_numpy(cs).cuda(), None if cand is None else torch.from_numpy(cand).cuda(),
                         ns, k, sel)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), oracle.select_columns(cs, cand, k, ns))


# ------------------------------------------------------------ quantiser --
@pytest.mark.parametrize("d,g,bits", [(128, 64, (8, 4, 2, 2)), (64, 32, (8, 4, 8, 2)),
                                      (128, 64, (32, 32, 4, 2))])
def test_quant_chain_bit_exact(d, g, bits):
    _say("quant", d, g, bits)
    rng = np.random.default_rng(d + len(bits))
    N, H = 777, 4
    levels = len(bits)
    x = [rng.standard_normal((N, H, d)).astype(np.float32)]
    for l in range(1, levels):
        x.append(x[-1] + (rng.standard_normal((N, H, d)) * 0.1 ** l).astype(np.float32))
    xb = [synth.f32_to_bf16_bits(a) for a in x]
    xf = [synth.bf16_bits_to_f32(a) for a in xb]
    rows = [np.arange(N, dtype=np.int32)]
    for l in range(1, levels):
        m = len(rows[-1]) * 2 // 3
        rows.append(np.sort(rng.choice(rows[-1], m, replace=False)).astype(np.int32))
    cache = fl.FlKvCache()
    cache.N, cache.H, cache.d, cache.g, cache.n_levels = N, H, d, g, levels
    keep = []
    xhk = xhv = None
    for l in range(levels):
        n = len(rows[l])
        kc = torch.zeros((n, H, d * bits[l] // 8), dtype=torch.uint8, device="cuda")
        vc = torch.zeros_like(kc)
        ks = torch.zeros((n, H, d // g), dtype=torch.float32, device="cuda")
        vs = torch.zeros_like(ks)
        L = cache.level[l]
        L.bits, L.n_rows = bits[l], n
        L.k_codes, L.v_codes, L.k_scale, L.v_scale = kc.data_ptr(), vc.data_ptr(), ks.data_ptr(), vs.data_ptr()
        if l > 0:
            rt = torch.from_numpy(rows[l]).cuda()
            slot = np.full(N, -1, np.int32); slot[rows[l]] = np.arange(n)
            st = torch.from_numpy(slot).cuda()
            L.rows, L.slot = rt.data_ptr(), st.data_ptr()
            keep += [rt, st]
        keep += [kc, vc, ks, vs]
        kn = to_dev(xb[l], "bf16")
        vn = to_dev(xb[(l + 1) % levels], "bf16")
        fl.fl_kv_residual_quant(cache, l, kn, vn)
        torch.cuda.synchronize()
        # oracle: same level on the same rows
        ck, sk, rk, xk = oracle.quantize_rows(xf[l][rows[l]], None if l == 0 else xhk[rows[l]], g, bits[l])
        cv, sv, rv, xv = oracle.quantize_rows(xf[(l + 1) % levels][rows[l]],
                                              None if l == 0 else xhv[rows[l]], g, bits[l])
        if bits[l] == 32:
            np.testing.assert_array_equal(kc.cpu().numpy().view(np.float32).reshape(rk.shape), rk)
            np.testing.assert_array_equal(vc.cpu().numpy().view(np.float32).reshape(rv.shape), rv)
        else:
            np.testing.assert_array_equal(kc.cpu().numpy(), oracle.pack_codes(ck, bits[l]))
            np.testing.assert_array_equal(vc.cpu().numpy(), oracle.pack_codes(cv, bits[l]))
            np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32), sk.view(np.uint32))
            np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32), sv.view(np.uint32))
        if l == 0:
            xhk, xhv = xk.copy(), xv.copy()
        else:
            xhk[rows[l]] = xk
            xhv[rows[l]] = xv


@pytest.mark.parametrize("d,g,bits,ties", [(128, 64, (4, 4, 4, 4), False), (64, 32, (4, 2, 8, 4), False),
                                           (128, 64, (4, 4, 2), True)])
def test_quant_asym_chain_bit_exact(d, g, bits, ties):
    """The paper's quantiser (App. E): codes, scales and offsets of every
    level bit-exact against the oracle, keys per channel over g packed rows
    (ragged last group: 777 rows, nested subsets), values per token.
    ties: bf16 inputs on a coarse grid (many equal values, signed zeros,
    constant groups)."""
    _say("quant asym", d, g, bits, ties)
    rng = np.random.default_rng(7 * d + len(bits))
    N, H = 777, 4
    levels = len(bits)
    x = [rng.standard_normal((N, H, d)).astype(np.float32)]
    for l in range(1, levels):
        x.append(x[-1] + (rng.standard_normal((N, H, d)) * 0.1 ** l).astype(np.float32))
    if ties:
        x = [np.round(a * 2) / 2 for a in x]
        x[0][:, 1, :] = -0.0                                  # constant (signed zero) groups
        x[0][5:70, 2, 3] = 1.5                                # a constant key channel
    xb = [synth.f32_to_bf16_bits(a.astype(np.float32)) for a in x]
    xf = [synth.bf16_bits_to_f32(a) for a in xb]
    rows = [np.arange(N, dtype=np.int32)]
    for l in range(1, levels):
        m = len(rows[-1]) * 2 // 3
        rows.append(np.sort(rng.choice(rows[-1], m, replace=False)).astype(np.int32))
    cache = fl.FlKvCache()
    cache.N, cache.H, cache.d, cache.g, cache.n_levels = N, H, d, g, levels
    cache.scheme = fl.FL_QUANT_ASYM
    keep = []
    xhk = xhv = None

    def buf(shape, dt):
        t = torch.zeros(shape, dtype=dt, device="cuda")
        keep.append(t)
        return t

    for l in range(levels):
        n = len(rows[l])
        t = fl.alloc_level(cache.level[l], n, H, d, g, bits[l], fl.FL_QUANT_ASYM, buf)
        if l > 0:
            rt = torch.from_numpy(rows[l]).cuda()
            slot = np.full(N, -1, np.int32); slot[rows[l]] = np.arange(n)
            st = torch.from_numpy(slot).cuda()
            cache.level[l].rows, cache.level[l].slot = rt.data_ptr(), st.data_ptr()
            keep += [rt, st]
        kn = to_dev(xb[l], "bf16")
        vn = to_dev(xb[(l + 1) % levels], "bf16")
        fl.fl_kv_residual_quant(cache, l, kn, vn)
        torch.cuda.synchronize()
        ck, sk, zk, xk = oracle.quantize_rows_asym(xf[l][rows[l]], None if l == 0 else xhk[rows[l]],
                                                   g, bits[l], True)
        cv, sv, zv, xv = oracle.quantize_rows_asym(xf[(l + 1) % levels][rows[l]],
                                                   None if l == 0 else xhv[rows[l]], g, bits[l], False)
        np.testing.assert_array_equal(t["k"].cpu().numpy(), oracle.pack_codes(ck, bits[l]))
        np.testing.assert_array_equal(t["v"].cpu().numpy(), oracle.pack_codes(cv, bits[l]))
        for got, want in ((t["ks"], sk), (t["kz"], zk), (t["vs"], sv), (t["vz"], zv)):
            np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
        if l == 0:
            xhk, xhv = xk.copy(), xv.copy()
        else:
            xhk[rows[l]] = xk
            xhv[rows[l]] = xv


# ------------------------------------------------------- whole loops --
def _chain(w, bits=None, mode=fl.FL_DEQ_AUTO, token_stat=fl.FL_TOKEN_STAT_ABS,
           col_stat=fl.FL_COL_STAT_MASS, quant=fl.FL_QUANT_ABSMAX):
    _say("chain", w.name, w.N, w.H, w.d, w.R, w.rho, w.kcols, bits or w.bits, "mode", mode,
         "stats", token_stat, col_stat, "quant", quant)
    inp = synth.generate(w)
    gres, _ = run_gpu(w, inp, mode=mode, bits=bits, token_stat=token_stat, col_stat=col_stat,
                      quant=quant)
    ores = run_oracle_lockstep(w, inp, gres, bits=bits, token_stat=token_stat, col_stat=col_stat,
                               quant=quant)
    rep = compare_chain(w, gres, ores, bits=bits, quant=quant)
    _say("  per-loop (r, rel-L2 out, rel-L2 lse):", [(r, f"{a[0]:.2e}", f"{b[0]:.2e}") for r, a, b in rep])
    return gres, ores


def test_tiny_workload_full():
    """The tiny case in full: 1 head x 64, N=256, R=2, fp32 inputs."""
    _chain(synth.WORKLOADS["tiny"])


@pytest.mark.parametrize("mode", [fl.FL_DEQ_ONCE, fl.FL_DEQ_IN_TILE])
def test_layer_recipe_pruning_ragged(mode):
    """Ouro-class layer recipe at N=1000 (ragged tiles), 8 heads (XCD-mapped
    grid), decreasing column budgets: cache rebuild at loops 2, 3 and 4 and
    column statistics at loops 1-3."""
    w = synth.WORKLOADS["layer4k"].scaled(N=1000, H=8, kcols=[1000, 300, 150, 100])
    _chain(w, mode=mode)


@pytest.mark.parametrize("mode", [fl.FL_DEQ_ONCE, fl.FL_DEQ_IN_TILE])
def test_prefill_recipe_small(mode):
    """32K-prefill recipe (fractions 1/.4/.2/.1, int4 then int2 residuals) at
    N=2048, 8 heads, 256 columns; both dequantisation placements."""
    w = synth.WORKLOADS["prefill32k"].scaled(N=2048, H=8, kcols=[2048, 256, 256, 256])
    _chain(w, mode=mode)


@pytest.mark.parametrize("mode", [fl.FL_DEQ_ONCE, fl.FL_DEQ_IN_TILE])
def test_head_dim_64_group_32(mode):
    w = synth.WORKLOADS["layer4k"].scaled(N=640, H=3, d=64, g=32, kcols=[640, 200, 120, 120],
                                          bits=[8, 4, 2, 4])
    _chain(w, mode=mode)


@pytest.mark.timeout(900)
def test_layer4k_full_shape():
    """The 4K layer workload at its own shape: N=4096, 16 x 128, R=4, 820
    active rows in each later loop, 512 columns including 4 sinks, int8 base
    and int4 residuals; every index set, code, output row and column
    statistic against the oracle in lock step."""
    _chain(synth.WORKLOADS["layer4k"])


def test_tiny_in_tile():
    _chain(synth.WORKLOADS["tiny"], mode=fl.FL_DEQ_IN_TILE)


def test_dense_reduction_raw():
    """rho = 1, k = all columns, unquantised residuals: every loop equals the
    oracle's dense causal attention (itself pinned to fp64 SDPA)."""
    w = synth.WORKLOADS["layer4k"].scaled(N=700, H=8, R=3, rho=[1.0, 1.0, 1.0],
                                          kcols=[700, 700, 700], bits=[8, 32, 32])
    _chain(w)


@pytest.mark.parametrize("mode", [fl.FL_DEQ_ONCE, fl.FL_DEQ_IN_TILE])
def test_stat_variants_chain(mode):
    """Relative token statistic and value-norm-weighted column statistic on
    the pruning layer recipe (ragged N, rebuilds at loops 2-4): active sets
    and column sets exact given the GPU's statistics, statistics within the
    usual bounds, outputs as for the default statistics."""
    w = synth.WORKLOADS["layer4k"].scaled(N=1000, H=8, kcols=[1000, 300, 150, 100], seed=31)
    _chain(w, mode=mode, token_stat=fl.FL_TOKEN_STAT_REL, col_stat=fl.FL_COL_STAT_VNORM)


def test_stat_variants_f32_d64():
    """The same variants with fp32 inputs (hi/lo operand gather) at d = 64."""
    w = synth.WORKLOADS["layer4k"].scaled(N=515, H=3, d=64, g=32, kcols=[515, 160, 90, 90],
                                          bits=[8, 4, 2, 4], dtype="f32", seed=32)
    _chain(w, token_stat=fl.FL_TOKEN_STAT_REL, col_stat=fl.FL_COL_STAT_VNORM)


def test_asym_quant_chain_prefill_recipe():
    """The paper's own quantiser (INT4 base and residuals, keys per channel,
    values per token) through whole loops on the 32K recipe at N = 2048:
    codes, scales and offsets bit-exact, outputs within the usual bounds."""
    w = synth.WORKLOADS["prefill32k"].scaled(N=2048, H=8, kcols=[2048, 256, 256, 256],
                                             bits=[4, 4, 4, 4], seed=33)
    _chain(w, quant=fl.FL_QUANT_ASYM)


def test_asym_quant_ragged_d64_f32():
    """Asymmetric scheme with d = 64, g = 32, ragged N (last key group short),
    2-bit residuals, fp32 inputs and pruning at every loop."""
    w = synth.WORKLOADS["layer4k"].scaled(N=515, H=3, d=64, g=32, kcols=[515, 160, 90, 60],
                                          bits=[4, 4, 2, 8], dtype="f32", seed=34)
    _chain(w, quant=fl.FL_QUANT_ASYM)
