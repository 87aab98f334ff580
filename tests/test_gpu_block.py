"""GPU parity of the token-sparse looped block (fl_block_step) against the
block oracle, on reduced recipes of the 8K/24-layer workload: ragged N, 1-2
layers, 3 loops with pruning column budgets.  Token and column selections
are fed the GPU's own statistics (index sets then compared exactly); hidden
states and per-layer attention outputs within rel-L2 1e-2 / max-abs 3e-2.

The projections feeding the quantiser are computed by two GEMM
implementations, so a K/V value can differ by a bf16 ulp or more (deeper
layers inherit ~1e-3 relative hidden-state differences) and move a code (the
random-init block changes its states by O(1) per loop, so the residual steps
are large).  The quantised run therefore checks that the oracle's own codes
agree with the GPU's (int8: under 15% differ, by at most 2; int4/int2: under
5%, by at most 1) and then rebuilds the cache from the GPU's stored codes
for the downstream comparison; codes themselves are bit-exact against the
oracle given identical inputs (attention-only tests).  The unquantised run
(raw residuals) compares the whole chain with no such substitution."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import block as ob
from sparse_attention_kv_amd import fl, synth

from gpu_block_chain import capture_block, oracle_block
from gpu_chain import assert_close, oracle_stat_names, to_dev

pytestmark = pytest.mark.gpu


def _workload(N=640, H=2, d=128, L=2, F=512, R=3):
    w = synth.WORKLOADS["block8k"].scaled(N=N, H=H, d=d, R=R, rho=[1.0, 0.5, 0.25][:R],
                                          kcols=[N, 256, 128][:R], bits=[8, 4, 2][:R])
    w.extra = dict(w.extra, layers=L, ffn=F, wstd=0.05)
    return w


@pytest.mark.parametrize("N,H,d,L,F,raw,variants,asym", [(640, 2, 128, 2, 512, False, False, False),
                                                         (389, 4, 64, 1, 256, False, False, False),
                                                         (512, 2, 128, 2, 256, True, False, False),
                                                         (450, 2, 128, 2, 256, False, True, False),
                                                         (600, 2, 128, 2, 256, False, False, True)])
def test_block_matches_oracle(N, H, d, L, F, raw, variants, asym):
    """variants: relative token statistic and value-norm-weighted columns;
    asym: the paper's own quantiser (INT4 base and residuals, keys per
    channel after RoPE, values per token)."""
    w = _workload(N, H, d, L, F)
    if raw:
        w.bits = [32, 32, 32]
    if asym:
        w.bits = [4, 4, 4]
    ts = fl.FL_TOKEN_STAT_REL if variants else fl.FL_TOKEN_STAT_ABS
    cs = fl.FL_COL_STAT_VNORM if variants else fl.FL_COL_STAT_MASS
    sched = w.sched()
    sched.update(oracle_stat_names(ts, cs))
    if asym:
        sched["quant"] = "asym"
    print("block", sched, "layers", L, "ffn", F, flush=True)
    inp = synth.generate(w)
    R = w.R
    n_act = [N]
    for r in range(1, R):
        n_act.append(oracle.active_count(w.rho[r], N, n_act[-1]))
    wdev = [{k: to_dev(v, "bf16") for k, v in lw.items()} for lw in inp["layers"]]
    run = fl.BlockRunner(N, H, d, w.g, R, w.n_sink, n_act, w.kcols, w.bits, wdev, F,
                         rope_theta=w.extra["theta"], norm_eps=w.extra["eps"], token_stat=ts,
                         col_stat=cs, quant=fl.FL_QUANT_ASYM if asym else fl.FL_QUANT_ABSMAX)
    G = capture_block(run, inp["h1"], n_act, w.kcols)
    for r in range(1, R + 1):
        print(f"  gpu loop {r}: n={len(G[r - 1]['active'])}", flush=True)
    res = oracle_block(inp, w, sched, G)
    for r in range(1, R + 1):
        g, o = G[r - 1], res[r - 1]
        np.testing.assert_array_equal(g["active"], o["active"], err_msg=f"loop {r} active")
        if r > 1:
            assert_close(g["stat"], o["stat"], f"loop {r} token statistic",
                         mabs=3e-2 * float(np.abs(o["stat"]).max()))
        for l in range(L):
            gl, ol = g["layers"][l], o["layers"][l]
            assert gl["k"] == ol["k"]
            if not raw:
                for kv in ("k", "v"):
                    mine = ol["level_" + kv]["codes"].astype(np.int16)
                    theirs = ob.unpack_codes(gl["kv"][kv], w.bits[r - 1], d,
                                             unsigned=asym).astype(np.int16)
                    diff = np.abs(mine - theirs)
                    frac = float(np.mean(diff != 0))
                    print(f"  loop {r} layer {l} {kv} codes: {frac:.2%} differ, max step {diff.max()}",
                          flush=True)
                    # int8's fine step (absmax/127) turns the ~1e-3 relative
                    # hidden-state differences of deeper layers into 1-2 step
                    # moves (a group's scale moves with its absmax element);
                    # int4/int2 steps are 18-60x coarser
                    fine = w.bits[r - 1] == 8
                    assert frac < (0.15 if fine else 0.05) and diff.max() <= (2 if fine else 1)
            e = assert_close(gl["out"], ol["out"], f"loop {r} layer {l} attention out")
            print(f"  loop {r} layer {l}: attention rel-L2 {e[0]:.2e} max-abs {e[1]:.2e}", flush=True)
        e = assert_close(g["h"], o["h"], f"loop {r} hidden state")
        print(f"  loop {r}: hidden rel-L2 {e[0]:.2e} max-abs {e[1]:.2e} (max |h| {np.abs(o['h']).max():.2f})",
              flush=True)
    inactive = np.setdiff1d(np.arange(N), G[-1]["active"])
    np.testing.assert_array_equal(G[-1]["h"][inactive], G[-2]["h"][inactive])
