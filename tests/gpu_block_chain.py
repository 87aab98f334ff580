"""Helpers for the looped-block GPU tests: run loops of ``fl_block_step``
through a BlockRunner, read back each loop's results, and run the block
oracle in lock step (fed the GPU's own statistics and stored cache codes, as
the block test module describes)."""
import numpy as np
import torch

from oracle import block as ob
from sparse_attention_kv_amd import synth


def capture_block(run, h1, n_act, kcols, loops=None):
    """Run loops 1..loops (default R) from hidden states h1 (numpy fp32)
    with active counts n_act; returns one record per loop."""
    R, L = run.R, run.L
    loops = loops or R
    run.set_active_counts(list(n_act))
    run.h.copy_(torch.from_numpy(np.ascontiguousarray(h1, np.float32)).cuda())
    G = []
    for r in range(1, loops + 1):
        run.step(r)
        torch.cuda.synchronize()
        rec = dict(active=run.active[r - 1][: n_act[r - 1]].cpu().numpy(), h=run.h.cpu().numpy())
        if r > 1:
            rec["stat"] = run.stat[: n_act[r - 2]].cpu().numpy().copy()
        rec["layers"] = []
        for l in range(L):
            lb = run.layer_bufs[l]
            k_used = run.layers[l].k_cur[r - 1]
            lr = dict(out=lb["out"].cpu().numpy()[rec["active"]],
                      lse=lb["lse"].cpu().numpy()[rec["active"]], k=k_used)
            if r < R and kcols[r] < k_used:
                lr["cstat"] = lb["col_stat"][r - 1][:, :k_used].cpu().numpy().copy()
            cb = lb["codes"][r - 1]
            rows = n_act[r - 1]
            lr["kv"] = {key: cb[key][:rows].cpu().numpy() for key in ("k", "v", "vs", "vz")
                        if key in cb}
            kg = -(-rows // run.g) if "kz" in cb else rows     # key groups of g rows (asym)
            lr["kv"]["ks"] = cb["ks"][:kg].cpu().numpy()
            if "kz" in cb:
                lr["kv"]["kz"] = cb["kz"][:kg].cpu().numpy()
            rec["layers"].append(lr)
        G.append(rec)
    return G


def oracle_block(inp, w, sched, G):
    """The block oracle on the same inputs, in lock step with the GPU run G
    (its statistics and stored codes); sched["rho"] must reproduce G's counts."""
    ov = {}
    L = len(inp["layers"])
    for r in range(2, len(G) + 1):
        ov[("stat", r)] = G[r - 1]["stat"]
        for l in range(L):
            if "cstat" in G[r - 2]["layers"][l]:
                ov[("cstat", r, l)] = G[r - 2]["layers"][l]["cstat"]
    for r in range(1, len(G) + 1):
        for l in range(L):
            ov[("kv", r, l)] = G[r - 1]["layers"][l]["kv"]
    layers = [{k: synth.bf16_bits_to_f32(v) for k, v in lw.items()} for lw in inp["layers"]]
    s = dict(sched)
    s["R"] = len(G)
    return ob.run_block(inp["h1"], layers, s, theta=w.extra["theta"], eps=w.extra["eps"],
                        override=ov, bf16_acts=True)
