"""GPU checks of the retention calibration (App. E of the FlashLoop paper):
the fp64 error reduction against numpy, and the calibration's decisions on a
small random-init block against the block oracle run in lock step with the
same schedules: every evaluated error within 1e-3 (+1%) of the oracle's,
and outside that band every accept / reject decision at the paper's 5% bound
the same by the oracle's error."""
import math

import numpy as np
import pytest
import torch

from sparse_attention_kv_amd import calibrate, fl, synth

from gpu_block_chain import capture_block, oracle_block
from gpu_chain import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 3, 4, 1027, 8192 * 2048 + 3])
def test_sq_err_matches_fp64(n):
    print("sq_err n", n, flush=True)
    rng = np.random.default_rng(n % 1000)
    x = rng.standard_normal(n).astype(np.float32)
    ref = (x + rng.standard_normal(n).astype(np.float32) * 0.01).astype(np.float32)
    xd, rd = torch.from_numpy(x).cuda(), torch.from_numpy(ref).cuda()
    out = torch.zeros(2, dtype=torch.float64, device="cuda")
    fl.fl_sq_err(xd, rd, out)
    got = out.cpu().numpy().copy()
    e2 = np.sum((x.astype(np.float64) - ref.astype(np.float64)) ** 2)
    r2 = np.sum(ref.astype(np.float64) ** 2)
    np.testing.assert_allclose(got, [e2, r2], rtol=1e-12)
    fl.fl_sq_err(xd, rd, out)
    assert np.array_equal(out.cpu().numpy(), got)        # deterministic
    fl.fl_sq_err(rd, rd, out)
    assert out.cpu().numpy()[0] == 0.0


def _block(N=384, H=2, d=64, L=1, F=256, R=3):
    w = synth.WORKLOADS["block8k"].scaled(N=N, H=H, d=d, R=R, rho=[1.0] * R,
                                          kcols=[N, 128, 64][:R], bits=[8, 4, 2][:R], seed=41)
    w.extra = dict(w.extra, layers=L, ffn=F, wstd=0.05)
    return w


def _oracle_err(w, inp, run, counts, G_ref_o):
    sched = w.sched()
    sched["rho"] = [c / w.N for c in counts] + [1.0] * (w.R - len(counts))
    full = list(counts) + [counts[-1]] * (w.R - len(counts))
    G = capture_block(run, inp["h1"], full, w.kcols, loops=len(counts))
    res = oracle_block(inp, w, sched, G)
    for r, rec in enumerate(res):
        np.testing.assert_array_equal(rec["active"], G[r]["active"])
    h = res[-1]["h"].astype(np.float64)
    href = G_ref_o[len(counts) - 1]["h"].astype(np.float64)
    return float(np.linalg.norm(h - href) / np.linalg.norm(href)), G[-1]["h"]


def test_calibration_decisions_match_oracle():
    w = _block()
    N, R = w.N, w.R
    inp = synth.generate(w)
    wdev = [{k: to_dev(v, "bf16") for k, v in lw.items()} for lw in inp["layers"]]
    run = fl.BlockRunner(N, w.H, w.d, w.g, R, w.n_sink, [N] * R, w.kcols, w.bits, wdev,
                         w.extra["ffn"], rope_theta=w.extra["theta"], norm_eps=w.extra["eps"],
                         row_capacity=[N] * R, capture_kv=True)
    h1 = torch.from_numpy(inp["h1"]).cuda()
    grid = [0.1 * i for i in range(1, 11)]
    tol = 0.05          # the paper's bound on the relative reconstruction error
    res = calibrate.calibrate_retention(run, h1, grid, tol=tol)
    print("bound", tol, "-> rho", res["rho"], "counts", res["n_active"],
          "errors", [f"{e:.4f}" for e in res["err"]], flush=True)
    # oracle reference (every token retained), in lock step with the GPU's
    sched_ref = w.sched()
    G_ref = capture_block(run, inp["h1"], [N] * R, w.kcols)
    ref_o = oracle_block(inp, w, sched_ref, G_ref)
    counts = [N]
    for r in range(2, R + 1):
        picked = res["n_active"][r - 1]
        for c, n, e_gpu in res["trials"][r]:
            e_o, _ = _oracle_err(w, inp, run, counts + [n], ref_o)
            print(f"  loop {r} rho {c:.1f} n {n}: gpu {e_gpu:.5f} oracle {e_o:.5f}", flush=True)
            assert abs(e_gpu - e_o) <= 1e-3 + 0.01 * e_o
            if abs(e_o - tol) <= 1e-3 + 0.01 * e_o:
                continue        # within the agreement band: either decision is valid
            # outside the band the oracle's error takes the GPU's decision
            assert (e_o < tol) == (e_gpu < tol)
            if n == picked and e_gpu < tol:
                assert e_o < tol
        counts.append(picked)
    # the accepted ratio is the smallest candidate under the bound
    for r in range(2, R + 1):
        tr = res["trials"][r]
        if res["err"][r - 1] < tol:
            assert tr[-1][1] == res["n_active"][r - 1]
            assert all(e >= tol for _, _, e in tr[:-1])
        assert res["n_active"][r - 1] <= res["n_active"][r - 2]
    assert math.isfinite(sum(res["err"]))
