"""Check mode (fl_set_checks): invalid index lists and statistics are
rejected with FL_ERR_INVALID_ARG before anything is enqueued (outputs stay
untouched), and valid runs are unchanged by the checks.  The invalid inputs
used here stay inside their buffers' bounds (unsorted or repeated positions,
NaN statistics), so no kernel could read out of bounds even unchecked."""
import numpy as np
import pytest
import torch

from sparse_attention_kv_amd import fl, synth

from gpu_chain import counts, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def checks():
    fl.fl_set_checks(True)
    yield
    fl.fl_set_checks(False)


def test_select_active_rejects_bad_inputs(checks):
    N, D = 300, 64
    h = torch.randn(N, D, device="cuda")
    stat = torch.zeros(N, device="cuda")
    act = torch.full((10,), -7, dtype=torch.int32, device="cuda")
    bad = torch.tensor([5, 3, 9, 11], dtype=torch.int32, device="cuda")       # unsorted
    with pytest.raises(fl.FlError) as e:
        fl.fl_select_active(h, h, bad, 2, stat, act)
    assert e.value.code == -1 and "cand" in str(e.value)
    dup = torch.tensor([1, 4, 4, 8], dtype=torch.int32, device="cuda")        # repeated
    with pytest.raises(fl.FlError):
        fl.fl_select_active(h, h, dup, 2, stat, act)
    s_in = torch.rand(N, device="cuda")
    s_in[17] = float("nan")
    with pytest.raises(fl.FlError) as e:
        fl.fl_select_active(None, None, None, 5, None, act, stat_in=s_in, N=N)
    assert "stat_in" in str(e.value)
    torch.cuda.synchronize()
    assert (act == -7).all().item()          # nothing was written


def test_select_columns_rejects_bad_inputs(checks):
    H, n, k = 2, 40, 12
    cs = torch.rand(H, n, device="cuda")
    cand = torch.arange(n, dtype=torch.int32, device="cuda").repeat(H, 1).contiguous()
    cand[1, 7], cand[1, 8] = cand[1, 8].item(), cand[1, 7].item()             # head 1 unsorted
    out = torch.full((H, k), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(fl.FlError) as e:
        fl.fl_select_columns(cs, cand, 4, k, out)
    assert "cand_cols row 1" in str(e.value)
    cand = torch.arange(n, dtype=torch.int32, device="cuda").repeat(H, 1).contiguous()
    cs[0, 3] = float("inf")
    with pytest.raises(fl.FlError) as e:
        fl.fl_select_columns(cs, cand, 4, k, out)
    assert "col_stat" in str(e.value)
    torch.cuda.synchronize()
    assert (out == -7).all().item()


def test_checked_chain_matches_unchecked():
    """A whole 4-loop chain under check mode (its own index sets pass) gives
    the same results as without it."""
    w = synth.WORKLOADS["layer4k"].scaled(N=700, H=2, R=4, rho=[1.0, 0.5, 0.3, 0.15],
                                          kcols=[700, 256, 160, 96])
    inp = synth.generate(w)
    dev = {k: [to_dev(a, "bf16") for a in inp[k]] for k in ("h", "q", "k", "v")}
    n_act = counts(w)
    outs = []
    for on in (False, True):
        fl.fl_set_checks(on)
        try:
            run = fl.LoopRunner(w.N, w.H, w.d, w.g, w.R, w.n_sink, n_act, w.kcols, w.bits)
            for r in range(1, w.R + 1):
                run.step(r, dev["h"][r - 1], dev["h"][r - 2] if r > 1 else None, dev["q"][r - 1],
                         dev["k"][r - 1], dev["v"][r - 1], dev["q"][r - 2] if r > 1 else None)
            torch.cuda.synchronize()
            outs.append((run.out.cpu().numpy().copy(), run.active[-1].cpu().numpy().copy()))
        finally:
            fl.fl_set_checks(False)
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    np.testing.assert_array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
