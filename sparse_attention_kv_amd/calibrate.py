"""Retention calibration of the looped block (FlashLoop paper, App. E
"Quantization Setting"): each sparse loop keeps the smallest retention ratio
whose hidden states stay within a relative reconstruction error (5%) of the
reference run.

The paper calibrates once per model on sampled text sequences; here the
block is the random-init one the caller built and the input is whatever
hidden states the caller passes (synthetic).  Readings of what the paper
leaves open:

  - reference: the same block, schedule of column budgets and quantisation,
    with every token retained in every loop, so the error isolates the
    retention decision being calibrated;
  - error after loop r: ||h_r - h_r^ref||_F / ||h_r^ref||_F over all N tokens
    (tokens inactive in loop r carry the state of the last loop that
    updated them);
  - greedy over loops: loop r takes the smallest candidate ratio (nested:
    at most loop r-1's count) whose error after loop r is below the bound,
    with loops 2..r-1 fixed at their calibrated ratios; if none qualifies it
    keeps loop r-1's count;
  - a ratio rho keeps ceil(rho * N) tokens (at least one, at most the
    previous loop's count).

Every loop runs through ``fl_block_step`` and every error through
``fl_sq_err``; this module only sequences the calls.
"""
from __future__ import annotations

import math

import torch

from . import fl


def retained_count(rho: float, N: int, n_prev: int) -> int:
    """Tokens kept at ratio rho: ceil(rho * N), clamped to [1, n_prev]."""
    n = int(math.ceil(rho * N - 1e-9))
    return max(1, min(n, n_prev))


class _ErrMeter:
    def __init__(self, n, device):
        self.out = torch.zeros(2, dtype=torch.float64, device=device)
        self.ws = torch.empty(fl.fl_workspace_size(fl.FL_WS_SQ_ERR, n), dtype=torch.uint8,
                              device=device)

    def rel(self, x, ref):
        fl.fl_sq_err(x, ref, self.out, self.ws)
        e2, r2 = self.out.tolist()
        return math.sqrt(e2 / r2) if r2 > 0 else (0.0 if e2 == 0 else math.inf)


def run_schedule(runner: "fl.BlockRunner", h1: torch.Tensor, n_active, loops=None):
    """Run loops 1..loops (default R) of ``runner`` from hidden states h1 with
    the given per-loop active counts; returns the hidden states after each
    loop (device copies)."""
    loops = loops or runner.R
    runner.set_active_counts(list(n_active) + [n_active[-1]] * (runner.R - len(n_active)))
    runner.h.copy_(h1)
    hs = []
    for r in range(1, loops + 1):
        runner.step(r)
        hs.append(runner.h.clone())
    return hs


def calibrate_retention(runner: "fl.BlockRunner", h1: torch.Tensor, grid, tol: float = 0.05):
    """Calibrate the per-loop retention ratios of ``runner`` (allocated with
    row_capacity N in every loop) on hidden states h1 [N][D] (fp32, device).

    grid: candidate ratios in (0, 1].  Returns dict(rho=[...], n_active=[...],
    err=[...] (error after each loop at the chosen schedule), trials={r:
    [(rho, count, err), ...]} in the order evaluated)."""
    N, R = runner.N, runner.R
    if any(c < N for c in runner.cap):
        raise ValueError("calibration needs a runner allocated with row_capacity N per loop")
    cands = sorted(set(float(g) for g in grid))
    if not cands or cands[0] <= 0 or cands[-1] > 1:
        raise ValueError("candidate ratios must lie in (0, 1]")
    meter = _ErrMeter(h1.numel(), h1.device)
    ref = run_schedule(runner, h1, [N] * R)
    rho, counts, errs = [1.0], [N], [0.0]
    trials = {}
    for r in range(2, R + 1):
        trials[r] = []
        pick = None
        seen = set()
        for c in cands:
            n = retained_count(c, N, counts[-1])
            if n in seen:
                continue
            seen.add(n)
            hs = run_schedule(runner, h1, counts + [n], loops=r)
            e = meter.rel(hs[-1], ref[r - 1])
            trials[r].append((c, n, e))
            if e < tol:
                pick = (c, n, e)
                break
        if pick is None:
            hs = run_schedule(runner, h1, counts + [counts[-1]], loops=r)
            pick = (rho[-1], counts[-1], meter.rel(hs[-1], ref[r - 1]))
        rho.append(pick[0]); counts.append(pick[1]); errs.append(pick[2])
    return dict(rho=rho, n_active=counts, err=errs, trials=trials)
