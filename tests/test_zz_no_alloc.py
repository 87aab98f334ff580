"""fl_sparse_loop_attn_noalloc (the library's per-GPU scratch as workspace)
against fl_sparse_loop_attn with a caller workspace, through the C ABI: two
calls in a row on identical inputs -- the 16 x 128 layer's sparse loop with
a cache rebuild and column statistics, then a smaller carried-cache call --
give bit-identical outputs; a call needing more than the scratch holds is
rejected with FL_ERR_WORKSPACE and writes nothing."""
import numpy as np
import pytest
import torch

from sparse_attention_kv_amd import fl, synth

from gpu_chain import counts, to_dev

pytestmark = pytest.mark.gpu


def _args(run, q, q_prev, active, n, sel, k, level, cache_op, st, col_stat):
    a = fl.FlAttnArgs()
    a.dtype, a.q, a.q_gathered = fl.FL_BF16, q.data_ptr(), 0
    a.active, a.n = active.data_ptr(), n
    a.sel, a.k = sel.data_ptr(), k
    a.sm = float(1.0 / np.sqrt(run.d))
    a.level, a.mode, a.cache_op = level, fl.FL_DEQ_AUTO, cache_op
    a.out, a.lse = st["out"].data_ptr(), st["lse"].data_ptr()
    a.mass_u, a.out_u = st["mass_u"].data_ptr(), st["out_u"].data_ptr()
    a.col_stat = col_stat.data_ptr() if col_stat is not None else None
    a.q_prev = q_prev.data_ptr() if q_prev is not None else None
    a.q_prev_gathered = 0
    a.col_stat_kind = fl.FL_COL_STAT_MASS
    return a


def _same(x, y, what):
    assert torch.equal(x.view(torch.int32), y.view(torch.int32)), what


def test_noalloc_matches_workspace_entry():
    w = synth.WORKLOADS["layer4k"].scaled(N=3000, H=16, R=3, rho=[1.0, 0.4, 0.2],
                                          kcols=[3000, 1024, 600], bits=[8, 4, 2])
    print("noalloc", w.sched(), flush=True)
    inp = synth.generate(w)
    dev = {k: [to_dev(a, "bf16") for a in inp[k]] for k in ("h", "q", "k", "v")}
    run = fl.LoopRunner(w.N, w.H, w.d, w.g, w.R, w.n_sink, counts(w), w.kcols, w.bits)

    def step(r):
        run.step(r, dev["h"][r - 1], dev["h"][r - 2] if r > 1 else None, dev["q"][r - 1],
                 dev["k"][r - 1], dev["v"][r - 1], dev["q"][r - 2] if r > 1 else None)

    step(1)
    step(2)
    snap2 = run.snapshot()          # the state loop 3 starts from
    step(3)                         # quantises level 2 and selects loop 3's columns
    torch.cuda.synchronize()
    act3, sel3, k3 = run.active[2], run.sel_used(3), run.k_used(3)
    assert k3 == 600 and run.k_used(2) == 1024
    ws = torch.empty(fl.fl_workspace_size(fl.FL_WS_SPARSE_ATTN, w.H, k3, w.d, len(act3)),
                     dtype=torch.uint8, device="cuda")

    def state_from(snap):
        return {key: snap["tensors"][key].cuda() for key in ("out", "lse", "mass_u", "out_u")}

    calls = [
        # loop 3 over its 600 columns with the pruned-column caches rebuilt
        # from loop 2 and column statistics for a next loop
        dict(n=len(act3), k=k3, sel=sel3, op=fl.FL_CACHE_REBUILD, stat=True),
        # then a smaller call: the first 200 active rows over each head's first
        # 256 selected columns, caches carried
        dict(n=200, k=256, sel=sel3[:, :256].contiguous(), op=fl.FL_CACHE_CARRY, stat=False),
    ]
    for i, c in enumerate(calls):
        print(f"  call {i}: n={c['n']} k={c['k']} cache_op={c['op']}", flush=True)
        outs = []
        for which in ("workspace", "noalloc"):
            st = state_from(snap2)
            cs = torch.full((w.H, c["k"]), -1.0, device="cuda") if c["stat"] else None
            a = _args(run, dev["q"][2], dev["q"][1], act3, c["n"], c["sel"], c["k"], 2, c["op"], st, cs)
            if which == "workspace":
                fl.fl_sparse_loop_attn(run.state.cache, a, ws)
            else:
                fl.fl_sparse_loop_attn_noalloc(run.state.cache, a)
            torch.cuda.synchronize()
            outs.append((st, cs))
        (s0, c0), (s1, c1) = outs
        for key in ("out", "lse", "mass_u", "out_u"):
            _same(s0[key], s1[key], f"call {i}: {key}")
        if c0 is not None:
            _same(c0, c1, f"call {i}: col_stat")
        rows = act3[: c["n"]].long()
        assert torch.isfinite(s1["out"][rows]).all() and torch.isfinite(s1["lse"][rows]).all()
        print(f"  call {i}: outputs bit-identical", flush=True)


def test_noalloc_rejects_oversize():
    """A dense call over 3000 columns and rows of 16 x 128 heads needs about
    104 MB of workspace, beyond the scratch: FL_ERR_WORKSPACE, nothing
    written."""
    N, H, d = 3000, 16, 128
    w = synth.WORKLOADS["layer4k"].scaled(N=N, H=H, R=1, rho=[1.0], kcols=[N], bits=[8])
    inp = synth.generate(w)
    run = fl.LoopRunner(N, H, d, w.g, 1, w.n_sink, [N], [N], [8])
    run.step(1, to_dev(inp["h"][0], "bf16"), None, to_dev(inp["q"][0], "bf16"),
             to_dev(inp["k"][0], "bf16"), to_dev(inp["v"][0], "bf16"), None)
    torch.cuda.synchronize()
    need = fl.fl_workspace_size(fl.FL_WS_SPARSE_ATTN, H, N, d, N)
    assert need > fl.NOALLOC_SCRATCH_BYTES
    st = {key: torch.full_like(getattr(run, key), 7.0) for key in ("out", "lse", "mass_u", "out_u")}
    a = fl.FlAttnArgs()
    a.dtype, a.q, a.q_gathered = fl.FL_BF16, to_dev(inp["q"][0], "bf16").data_ptr(), 0
    a.active, a.n, a.sel, a.k = run.active[0].data_ptr(), N, None, N
    a.sm, a.level, a.mode, a.cache_op = float(1 / np.sqrt(d)), 0, fl.FL_DEQ_AUTO, fl.FL_CACHE_ZERO
    a.out, a.lse, a.mass_u, a.out_u = (st[k].data_ptr() for k in ("out", "lse", "mass_u", "out_u"))
    with pytest.raises(fl.FlError) as e:
        fl.fl_sparse_loop_attn_noalloc(run.state.cache, a)
    assert e.value.code == -3 and "workspace" in str(e.value)
    torch.cuda.synchronize()
    assert all((t == 7.0).all().item() for t in st.values())
