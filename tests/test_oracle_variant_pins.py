"""Pins of the oracle's statistic variants (no GPU).

App. E of the FlashLoop paper quantises base states and residuals with INT4
asymmetric min/max groups of 64: keys after RoPE per channel, values per
token (the paper's own quantiser, an alternative to the absmax one).

Sec. 4.1 of the FlashLoop paper ranks tokens by their *normalised*
hidden-state change; the plain reading is the change relative to the previous
loop's state, ||h_r - h_{r-1}|| / ||h_{r-1}||.  Sec. 4.2 ranks columns by an
"attention contribution" statistic from the previous loop; besides the column
probability mass, the oracle offers the mass weighted by the norm of the
column's value vector, i.e. the size of the column's contribution to the
loop's outputs.  Each pin names the mistake it would catch.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.block import dequant_rows_asym, unpack_codes
from oracle.loop import run_prefill
from sparse_attention_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------- relative statistic --
def test_rel_delta_closed_form():
    """3-4-5 triangles and the zero-state cases.  Catches: dividing by the
    current state instead of the previous one, a squared ratio, a missing
    sqrt on either norm."""
    prev = np.array([[3, 4, 0, 0], [0, 0, 0, 1], [0, 0, 0, 0], [0, 0, 0, 0],
                     [6, 8, 0, 0]], np.float32)
    cur = np.array([[3, 4, 6, 8], [0, 0, 0, 3], [0, 0, 0, 0], [0, 5, 0, 0],
                    [6, 8, 0, 0]], np.float32)
    got = oracle.delta_norm(cur, prev, relative=True)
    np.testing.assert_array_equal(got, [2, 2, 0, np.inf, 0])
    # candidate rows are honoured
    np.testing.assert_array_equal(
        oracle.delta_norm(cur, prev, cand=np.array([4, 1], np.int32), relative=True), [0, 2])
    # absolute statistic of the same rows for contrast: 10, 2, 0, 5, 0
    np.testing.assert_array_equal(oracle.delta_norm(cur, prev), [10, 2, 0, 5, 0])


def test_rel_delta_scale_invariant():
    """Scaling both states by a power of two leaves the ratio bit-identical;
    scaling only the current state's change scales the ratio.  Catches:
    normalising by D or by a global constant instead of the row's own norm."""
    rng = np.random.default_rng(4)
    a = rng.standard_normal((40, 256)).astype(np.float32)
    b = rng.standard_normal((40, 256)).astype(np.float32)
    base = oracle.delta_norm(a, b, relative=True)
    for s in (2.0 ** -7, 0.5, 8.0, 2.0 ** 20):
        np.testing.assert_array_equal(
            oracle.delta_norm(a * np.float32(s), b * np.float32(s), relative=True), base)
    ref = (np.linalg.norm(a.astype(np.float64) - b, axis=1) / np.linalg.norm(b.astype(np.float64),
                                                                           axis=1))
    np.testing.assert_allclose(base, ref, rtol=3e-6)


def test_rel_delta_reduces_to_absolute_ranking():
    """When every previous state has the same norm (sign flips and
    permutations of one vector), the relative statistic is the absolute one
    over a constant, so both select the same tokens.  Catches a ratio that
    depends on anything but the row's own previous norm."""
    rng = np.random.default_rng(8)
    D, N = 64, 300
    v = rng.standard_normal(D).astype(np.float32)
    prev = np.stack([rng.permutation(v) * np.where(rng.random(D) < 0.5, -1, 1)
                     for _ in range(N)]).astype(np.float32)
    cur = prev + rng.standard_normal((N, D)).astype(np.float32) * \
        rng.uniform(0.01, 1.0, (N, 1)).astype(np.float32)
    ab = oracle.delta_norm(cur, prev)
    rl = oracle.delta_norm(cur, prev, relative=True)
    pos = np.arange(N, dtype=np.int32)
    for n_sel in (1, 30, 150):
        np.testing.assert_array_equal(oracle.top_select(rl, n_sel, pos),
                                      oracle.top_select(ab, n_sel, pos))
    np.testing.assert_allclose(rl * np.linalg.norm(v.astype(np.float64)), ab, rtol=3e-6)


def test_rel_delta_ranks_small_states_up():
    """A token with a small absolute but large relative change wins under the
    relative statistic and loses under the absolute one."""
    prev = np.array([[100, 0], [1, 0]], np.float32)
    cur = np.array([[100, 5], [1, 1]], np.float32)     # abs 5 vs 1; rel 0.05 vs 1
    pos = np.arange(2, dtype=np.int32)
    assert list(oracle.top_select(oracle.delta_norm(cur, prev), 1, pos)) == [0]
    assert list(oracle.top_select(oracle.delta_norm(cur, prev, relative=True), 1, pos)) == [1]


# ----------------------------------------- value-weighted column statistic --
def _inputs(N, H=2, d=64, seed=3):
    w = synth.WORKLOADS["layer4k"].scaled(N=N, H=H, d=d, R=2, seed=seed, dtype="f32",
                                          rho=[1.0, 1.0], kcols=[N, N], bits=[32, 32], g=32)
    return synth.as_f32_inputs(synth.generate(w))


def test_vnorm_stat_unit_values_equal_mass():
    """One-hot value vectors have norm exactly 1, so the weighted statistic
    is the mass statistic bit for bit; doubling every value vector doubles it
    exactly; scaling one column's values by 4 scales only that column."""
    N, H, d = 70, 2, 64
    x = _inputs(N, H, d)
    q, k = x["q"][0], x["k"][0]
    sm = np.float32(1 / 8)
    rng = np.random.default_rng(2)
    v = np.zeros((N, H, d), np.float32)
    v[np.arange(N)[:, None], np.arange(H)[None], rng.integers(0, d, (N, H))] = \
        np.where(rng.random((N, H)) < 0.5, -1.0, 1.0)
    _, lse = oracle.attend(q, k, v, None, None, sm)
    mass = oracle.column_stats(q, k, None, None, lse, sm)
    np.testing.assert_array_equal(oracle.column_stats(q, k, None, None, lse, sm, vhat=v), mass)
    np.testing.assert_array_equal(oracle.column_stats(q, k, None, None, lse, sm, vhat=2 * v),
                                  2 * mass)
    v4 = v.copy(); v4[17] *= 4
    got = oracle.column_stats(q, k, None, None, lse, sm, vhat=v4)
    want = mass.copy(); want[:, 17] *= 4
    np.testing.assert_array_equal(got, want)


def test_vnorm_stat_is_output_contribution():
    """fp64 brute force: the weighted statistic of column j equals the sum
    over rows of the norm of that column's term P(i,j) v(j) in the row's
    output (computed as vectors, not as mass times norm).  Catches a norm
    over the wrong axis (keys, or the token's row) or a squared norm."""
    N, H, d = 60, 2, 64
    x = _inputs(N, H, d, seed=6)
    q, k, v = x["q"][0], x["k"][0], x["v"][0]
    sm = np.float32(1 / 8)
    _, lse = oracle.attend(q, k, v, None, None, sm)
    got = oracle.column_stats(q, k, None, None, lse, sm, vhat=v)
    s = np.einsum("ihd,jhd->hij", q.astype(np.float64), k.astype(np.float64)) * np.float64(sm)
    s = np.where(np.tril(np.ones((N, N), bool))[None], s, -np.inf)
    P = np.exp(s - s.max(axis=2, keepdims=True))
    P /= P.sum(axis=2, keepdims=True)
    term = P[..., None] * np.transpose(v.astype(np.float64), (1, 0, 2))[:, None, :, :]
    want = np.linalg.norm(term, axis=3).sum(axis=1)
    np.testing.assert_allclose(got, want, rtol=3e-5, atol=1e-7)
    # one token: its only column carries probability 1
    one = oracle.column_stats(q[:1], k[:1], None, None, lse[:1], sm, vhat=v[:1])
    np.testing.assert_allclose(one[:, 0], np.linalg.norm(v[0].astype(np.float64), axis=1),
                               rtol=1e-6)


def test_loop_variants_select_by_their_statistic():
    """Whole-loop wiring: with token_stat = "rel" the loop-2 active set is the
    brute-force top by the fp64 relative change, and with col_stat = "vnorm"
    the loop-2 columns are the sinks plus the brute-force top by fp64
    mass x ||v||.  Catches a driver that silently keeps the default
    statistics."""
    N, H, d = 96, 2, 64
    w = synth.WORKLOADS["layer4k"].scaled(N=N, H=H, d=d, R=2, seed=21, dtype="f32",
                                          rho=[1.0, 0.3], kcols=[N, 24], bits=[32, 32], g=32)
    x = synth.as_f32_inputs(synth.generate(w))
    sched = w.sched()
    sched.update(token_stat="rel", col_stat="vnorm")
    res = run_prefill(x["h"], x["q"], x["k"], x["v"], sched)
    h1, h0 = x["h"][1].astype(np.float64), x["h"][0].astype(np.float64)
    rel = np.linalg.norm(h1 - h0, axis=1) / np.linalg.norm(h0, axis=1)
    n2 = oracle.active_count(0.3, N, N)
    np.testing.assert_array_equal(res[1]["active"], np.sort(np.argsort(-rel, kind="stable")[:n2]))
    q, k, v = (a[0].astype(np.float64) for a in (x["q"], x["k"], x["v"]))
    s = np.einsum("ihd,jhd->hij", q, k) / 8.0
    s = np.where(np.tril(np.ones((N, N), bool))[None], s, -np.inf)
    P = np.exp(s - s.max(axis=2, keepdims=True))
    P /= P.sum(axis=2, keepdims=True)
    c = P.sum(axis=1) * np.linalg.norm(v, axis=2).T          # [H][N]
    n_sink = sched["n_sink"]
    for hh in range(H):
        top = n_sink + np.argsort(-c[hh, n_sink:], kind="stable")[:24 - n_sink]
        want = np.sort(np.concatenate([np.arange(n_sink), top]))
        np.testing.assert_array_equal(res[1]["sel"][hh], want)


# ------------------------------------------------- the paper's quantiser --
def _asym_golden():
    rows = []
    with open(os.path.join(GOLDEN, "quant_asym_groups.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            b, x, s, z, c, p = [t.strip() for t in line.split("|")]
            rows.append((int(b), np.array(x.split(), np.float32), np.float32(float(Fraction(s))),
                         np.float32(z), np.array(c.split(), np.uint8),
                         bytes.fromhex(p.replace(" ", ""))))
    return rows


def test_asym_golden():
    """Hand-worked groups (tests/golden/quant_asym_groups.txt): offset = min,
    scale = range/qmax, ties to even, the fp32 rounding of a 1/15 scale,
    unsigned packing.  Catches: symmetric scale, signed codes, offset = max or
    mean, floor/ceil rounding, qmax = 2^(b-1)-1."""
    rows = _asym_golden()
    assert len(rows) == 7
    for bits, x, s, z, codes, packed in rows:
        gc, gs, gz = oracle.quant_asym_group(x, bits)
        assert gs == s and gz == z, (bits, x, gs, gz)
        np.testing.assert_array_equal(gc, codes)
        assert oracle.pack_codes(codes, bits).tobytes() == packed


def test_asym_signed_zero_stored_as_plus_zero():
    """Groups of signed zeros: offset and scale are +0 whatever the order."""
    for x in ([0.0, -0.0], [-0.0, 0.0, -0.0], [-0.0, -0.0]):
        c, s, z = oracle.quant_asym_group(np.array(x, np.float32), 4)
        assert np.float32(s).view(np.uint32) == 0 and np.float32(z).view(np.uint32) == 0
        assert not c.any()


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_asym_bounds_random(bits):
    """|code*s + z - x| <= s/2 (plus fp32 rounding of the two steps); the
    minimum reconstructs exactly and maps to 0, the maximum to qmax."""
    rng = np.random.default_rng(bits)
    qmax = (1 << bits) - 1
    for _ in range(200):
        n = int(rng.integers(2, 80))
        x = (rng.standard_normal(n) * np.exp(rng.normal(0, 2))).astype(np.float32)
        c, s, z = oracle.quant_asym_group(x, bits)
        assert c.max() <= qmax
        deq = (c.astype(np.float32) * s).astype(np.float32) + z
        err = np.abs(deq.astype(np.float64) - x.astype(np.float64))
        assert np.all(err <= s / 2 + 4 * np.spacing(np.abs(x).max()))
        assert z == x.min() and c[np.argmin(x)] == 0 and c[np.argmax(x)] == qmax


def test_asym_axes():
    """Keys per channel over g consecutive rows (last group shorter), values
    per token over g channels: each group equals the single-group routine
    applied by hand to that slice; a channel constant over a key group (or a
    value group constant within a token) reproduces exactly.  Catches a
    transposed group axis or wrong group boundaries."""
    rng = np.random.default_rng(12)
    n, H, d, g = 150, 2, 64, 32
    x = rng.standard_normal((n, H, d)).astype(np.float32)
    x[:, 1, 5] = 2.25                                # constant key channel
    x[7, 0, 32:64] = -1.0                            # constant value group
    kc, ks, kz, kh = oracle.quantize_rows_asym(x, None, g, 4, per_channel=True)
    assert ks.shape == (5, H, d) and kz.shape == (5, H, d)
    for grp in range(5):
        r0, r1 = grp * g, min(n, grp * g + g)
        for h in range(H):
            for ch in (0, 5, 31, 63):
                c, s, z = oracle.quant_asym_group(x[r0:r1, h, ch], 4)
                np.testing.assert_array_equal(kc[r0:r1, h, ch], c)
                assert ks[grp, h, ch] == s and kz[grp, h, ch] == z
    np.testing.assert_array_equal(kh[:, 1, 5], 2.25)
    vc, vs, vz, vh = oracle.quantize_rows_asym(x, None, g, 4, per_channel=False)
    assert vs.shape == (n, H, d // g)
    for row in (0, 7, 149):
        for h in range(H):
            for q in range(d // g):
                c, s, z = oracle.quant_asym_group(x[row, h, q * g:(q + 1) * g], 4)
                np.testing.assert_array_equal(vc[row, h, q * g:(q + 1) * g], c)
                assert vs[row, h, q] == s and vz[row, h, q] == z
    np.testing.assert_array_equal(vh[7, 0, 32:64], -1.0)


def test_asym_residual_chain():
    """A residual level quantises x_new - xhat_prev and reconstructs
    xhat_prev + (code*s + z): its error is bounded by half the residual
    group's step; unpacking the packed codes and dequantising them with the
    block oracle's independent routine gives the same xhat bit for bit."""
    rng = np.random.default_rng(3)
    n, H, d, g = 100, 2, 64, 32
    x1 = rng.standard_normal((n, H, d)).astype(np.float32)
    x2 = (x1 + 0.05 * rng.standard_normal((n, H, d))).astype(np.float32)
    for pc in (True, False):
        _, _, _, xh1 = oracle.quantize_rows_asym(x1, None, g, 4, pc)
        c, s, z, xh2 = oracle.quantize_rows_asym(x2, xh1, g, 2, pc)
        step = np.repeat(s, g, axis=0)[:n] if pc else np.repeat(s, g, axis=-1)
        err = np.abs(xh2.astype(np.float64) - x2)
        assert np.all(err <= step / 2 + 1e-6)
        packed = oracle.pack_codes(c, 2)
        np.testing.assert_array_equal(unpack_codes(packed, 2, d, unsigned=True), c)
        np.testing.assert_array_equal(dequant_rows_asym(packed, s, z, 2, g, xh1, pc), xh2)


def test_residual_beats_direct_when_updates_are_small():
    """The observation behind residual storage (Sec. 3.3, Fig. 2(c)): when a
    loop changes the states by a small amount, quantising the change against
    the previous loop's reconstruction leaves a much smaller relative error
    than quantising the new states directly with the same scheme."""
    rng = np.random.default_rng(5)
    n, H, d, g = 256, 2, 128, 64
    x1 = rng.standard_normal((n, H, d)).astype(np.float32)
    x2 = (x1 + 0.02 * rng.standard_normal((n, H, d))).astype(np.float32)
    for pc in (True, False):
        _, _, _, xh1 = oracle.quantize_rows_asym(x1, None, g, 4, pc)
        _, _, _, res = oracle.quantize_rows_asym(x2, xh1, g, 4, pc)
        _, _, _, direct = oracle.quantize_rows_asym(x2, None, g, 4, pc)
        e_res = np.linalg.norm(res - x2) / np.linalg.norm(x2)
        e_dir = np.linalg.norm(direct - x2) / np.linalg.norm(x2)
        assert e_res < 0.1 * e_dir, (pc, e_res, e_dir)


def test_asym_driver_unchanged_inputs_keep_output():
    """Loop driver with the paper's quantiser: feeding loop 1's dequantised
    K/V as the later loops' K/V makes every residual group constant zero
    (reproduced exactly), so each pruned sparse loop restores loop 1's
    output; codes of the zero residuals are all 0."""
    N, H, d = 120, 2, 64
    w = synth.WORKLOADS["layer4k"].scaled(N=N, H=H, d=d, R=3, seed=9, dtype="f32",
                                          rho=[1.0, 0.5, 0.25], kcols=[N, 40, 20], bits=[4, 4, 2],
                                          g=32)
    x = synth.as_f32_inputs(synth.generate(w))
    _, _, _, kh = oracle.quantize_rows_asym(x["k"][0], None, 32, 4, True)
    _, _, _, vh = oracle.quantize_rows_asym(x["v"][0], None, 32, 4, False)
    sched = w.sched()
    sched["quant"] = "asym"
    res = run_prefill(x["h"], [x["q"][0]] * 3, [x["k"][0], kh, kh], [x["v"][0], vh, vh], sched)
    assert res[1]["sel_changed"] and res[2]["sel_changed"]
    for rec in res[1:]:
        np.testing.assert_allclose(rec["out"], res[0]["out"][rec["active"]], rtol=0, atol=3e-6)
        assert not rec["level_k"]["codes"].any() and not rec["level_v"]["codes"].any()
        assert rec["level_k"]["scales"].shape[0] == (len(rec["active"]) + 31) // 32
