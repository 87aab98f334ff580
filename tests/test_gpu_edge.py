"""GPU parity at the method's degenerate and extreme cases, each through the
whole loop chain in lock step with the oracle (index sets and codes exact,
outputs within the usual bounds):

  * a single token (N = 1), and a prefix shorter than one column tile;
  * the smallest column budget (the sinks plus one column);
  * a single active token in every sparse loop;
  * all-equal token statistics (ties: the lowest positions are kept);
  * ternary (int2) and int8 residuals at every sparse loop;
  * the widest head layout (H * d = 8192);
  * batched decode of one sequence with a 5-token prefix."""
import numpy as np
import pytest

from sparse_attention_kv_amd import synth

from gpu_chain import compare_chain, run_gpu, run_oracle_lockstep
from gpu_decode_chain import check_sequence, run_decode_gpu

pytestmark = pytest.mark.gpu


def _chain(w, inp=None):
    print("edge", w.N, w.H, w.d, w.R, w.rho, w.kcols, w.bits, flush=True)
    inp = inp or synth.generate(w)
    gres, _ = run_gpu(w, inp)
    ores = run_oracle_lockstep(w, inp, gres)
    compare_chain(w, gres, ores)
    return gres


def _layer(**kw):
    return synth.WORKLOADS["layer4k"].scaled(**kw)


def test_single_token():
    g = _chain(_layer(N=1, H=2, R=3, rho=[1.0, 1.0, 1.0], kcols=[1, 1, 1], bits=[8, 4, 2]))
    assert all(len(r["active"]) == 1 for r in g)


def test_prefix_shorter_than_a_tile():
    _chain(_layer(N=7, H=3, R=3, rho=[1.0, 0.5, 0.3], kcols=[7, 6, 5], bits=[8, 4, 4]))


def test_minimal_column_budget():
    g = _chain(_layer(N=300, H=2, R=3, rho=[1.0, 0.5, 0.5], kcols=[300, 5, 5], bits=[8, 4, 2]))
    assert g[1]["k"] == 5 and g[1]["sel"].shape == (2, 5)


def test_single_active_token():
    g = _chain(_layer(N=333, H=2, R=4, rho=[1.0, 1e-9, 1e-9, 1e-9], kcols=[333, 64, 32, 32],
                      bits=[8, 4, 2, 2]))
    assert [len(r["active"]) for r in g] == [333, 1, 1, 1]


def test_all_statistics_tied():
    w = _layer(N=200, H=2, R=3, rho=[1.0, 0.3, 0.3], kcols=[200, 64, 64], bits=[8, 4, 4])
    inp = synth.generate(w)
    inp["h"] = [inp["h"][0]] * 3          # no token changes: every statistic is 0
    g = _chain(w, inp)
    n2 = len(g[1]["active"])
    np.testing.assert_array_equal(g[1]["active"], np.arange(n2))   # ties -> lowest positions
    np.testing.assert_array_equal(g[2]["active"], np.arange(len(g[2]["active"])))


@pytest.mark.parametrize("bits", [(8, 2, 2, 2), (8, 8, 8, 8)])
def test_residual_widths(bits):
    _chain(_layer(N=513, H=4, R=4, rho=[1.0, 0.5, 0.25, 0.2], kcols=[513, 128, 96, 64],
                  bits=list(bits), seed=41))


def test_widest_heads():
    _chain(_layer(N=200, H=64, d=128, R=2, rho=[1.0, 0.5], kcols=[200, 100], bits=[8, 4], seed=42))


def test_decode_one_sequence_short_prefix():
    w = synth.WORKLOADS["decode64x8k"].scaled(N=5, H=2, d=128, g=64, R=3, kcols=[5, 5, 5],
                                              bits=[8, 4, 4], rho=[1.0, 0.6, 0.4], seed=43)
    w.extra = dict(B=1)
    gres, kept, run = run_decode_gpu(w, keep={0}, threads=1)
    check_sequence(w, 0, kept[0], gres, run)
