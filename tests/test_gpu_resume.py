"""Checkpoint / resume of the loop state: after any loop r the whole state
(cache levels, index sets, column statistics, per-row output / lse / M_U /
O_U, and the host bookkeeping of fl_loop_state) is snapshotted to the host;
restoring it -- into the same runner after it has run further, or into a
fresh runner -- and running loop r + 1 gives the uninterrupted run's state
bit for bit.  Budgets shrink every loop, so each resumed loop selects
columns and rebuilds the pruned-column caches."""
import numpy as np
import pytest
import torch

from sparse_attention_kv_amd import fl, synth

from gpu_chain import counts, to_dev

pytestmark = pytest.mark.gpu


def _equal(a, b, tag):
    assert a["k_cur"] == b["k_cur"] and a["sel_used"] == b["sel_used"], tag
    assert a["levels"] == b["levels"] and a["n_levels"] == b["n_levels"], tag
    for k, t in a["tensors"].items():
        u = b["tensors"][k]
        assert torch.equal(t.view(torch.uint8) if t.dtype != torch.uint8 else t,
                           u.view(torch.uint8) if u.dtype != torch.uint8 else u), f"{tag}: {k}"


@pytest.mark.parametrize("quant", [fl.FL_QUANT_ABSMAX, fl.FL_QUANT_ASYM])
def test_resume_bit_exact(quant):
    w = synth.WORKLOADS["layer4k"].scaled(N=900, H=4, R=4, rho=[1.0, 0.5, 0.3, 0.15],
                                          kcols=[900, 300, 200, 120],
                                          bits=[8, 4, 2, 2] if quant == fl.FL_QUANT_ABSMAX else [4] * 4)
    print("resume", w.sched(), "quant", quant, flush=True)
    inp = synth.generate(w)
    dev = {k: [to_dev(a, "bf16") for a in inp[k]] for k in ("h", "q", "k", "v")}
    n_act = counts(w)

    def make():
        return fl.LoopRunner(w.N, w.H, w.d, w.g, w.R, w.n_sink, n_act, w.kcols, w.bits, quant=quant)

    def step(run, r):
        run.step(r, dev["h"][r - 1], dev["h"][r - 2] if r > 1 else None, dev["q"][r - 1],
                 dev["k"][r - 1], dev["v"][r - 1], dev["q"][r - 2] if r > 1 else None)

    A = make()
    snaps = {}
    for r in range(1, w.R + 1):
        step(A, r)
        snaps[r] = A.snapshot()
    for r in range(1, w.R):
        # the same runner, whose state has moved on to loop R
        A.restore(snaps[r])
        step(A, r + 1)
        _equal(A.snapshot(), snaps[r + 1], f"same runner, loop {r + 1}")
        # a fresh runner of the same configuration
        B = make()
        B.restore(snaps[r])
        step(B, r + 1)
        _equal(B.snapshot(), snaps[r + 1], f"fresh runner, loop {r + 1}")
        print(f"  loop {r + 1} resumed from the loop-{r} snapshot: bit-identical", flush=True)
