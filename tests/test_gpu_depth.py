"""GPU parity at depth: 32 loops with kept fractions and column budgets that
shrink every loop (a cache rebuild at nearly every loop, 32 cache levels,
int4 then int2 residuals), against the oracle in lock step (index sets,
codes and column sets exact; outputs, lse and caches within the usual
bounds).  Reduced sizes of the 32-loop, 8K recipe."""
import sys

import pytest

from sparse_attention_kv_amd import fl, synth

from gpu_chain import compare_chain, run_gpu, run_oracle_lockstep

pytestmark = pytest.mark.gpu


def _chain(w, quant=fl.FL_QUANT_ABSMAX, mode=fl.FL_DEQ_AUTO):
    print("depth chain", w.N, w.H, w.R, "k", w.kcols[:4], "...", w.kcols[-1], "bits", w.bits[:3],
          "quant", quant, "mode", mode, flush=True)
    inp = synth.generate(w)
    gres, _ = run_gpu(w, inp, quant=quant, mode=mode)
    ores = run_oracle_lockstep(w, inp, gres, quant=quant)
    rep = compare_chain(w, gres, ores, quant=quant)
    worst = max(rep, key=lambda t: t[1][0])
    print(f"  worst loop {worst[0]}: out rel-L2 {worst[1][0]:.2e}", flush=True)
    sys.stdout.flush()


def test_depth32_small():
    _chain(synth.WORKLOADS["depth32x8k"].scaled(N=600, H=4))


def test_depth32_small_in_tile():
    """In-tile dequantisation through 32 levels: the LDS-DMA kernel while a
    tile's planes fit its staging buffer (about the first 8 loops here),
    then the register-staged kernel."""
    _chain(synth.WORKLOADS["depth32x8k"].scaled(N=600, H=4), mode=fl.FL_DEQ_IN_TILE)


@pytest.mark.timeout(600)
def test_depth32_medium():
    _chain(synth.WORKLOADS["depth32x8k"].scaled(N=2048, H=8))


def test_depth32_asym():
    w = synth.WORKLOADS["depth32x8k"]
    _chain(w.scaled(N=700, H=2, bits=[4] * w.R), quant=fl.FL_QUANT_ASYM)
