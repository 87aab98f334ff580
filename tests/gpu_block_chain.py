"""Helpers for the looped-block GPU tests: run loops of ``fl_block_step``
through a BlockRunner, read back each loop's results, and run the block
oracle in lock step.

Lock step means the oracle is fed two kinds of values from the GPU run, each
the input of a decision that must come out identically on both sides:
  * the GPU's fp32 statistic buffers, for the token and column selections
    (index sets are then unique and compared exactly);
  * the GPU's pre-quantisation keys (after RoPE) and values of each level,
    which the oracle's own quantiser then quantises (codes and scales are
    then compared bit for bit).  The oracle's own keys and values are
    checked against these first, within the attention tolerance.
Everything else -- the oracle's cache, queries, attention, projections and
residual stream -- is the oracle's own."""
import numpy as np
import torch

from oracle import block as ob
from sparse_attention_kv_amd import synth


def capture_block(run, h1, n_act, kcols, loops=None):
    """Run loops 1..loops (default R) from hidden states h1 (numpy fp32)
    with active counts n_act; returns one record per loop.  The runner must
    have been built with capture_kv=True."""
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
        rows = n_act[r - 1]
        for l in range(L):
            lb = run.layer_bufs[l]
            k_used = run.layers[l].k_cur[r - 1]
            lr = dict(out=lb["out"].cpu().numpy()[rec["active"]],
                      lse=lb["lse"].cpu().numpy()[rec["active"]], k=k_used)
            if r < R and kcols[r] < k_used:
                lr["cstat"] = lb["col_stat"][r - 1][:, :k_used].cpu().numpy().copy()
            cb = lb["codes"][r - 1]
            lr["kv"] = {key: cb[key][:rows].cpu().numpy() for key in ("k", "v", "vs", "vz")
                        if key in cb}
            kg = -(-rows // run.g) if "kz" in cb else rows     # key groups of g rows (asym)
            lr["kv"]["ks"] = cb["ks"][:kg].cpu().numpy()
            if "kz" in cb:
                lr["kv"]["kz"] = cb["kz"][:kg].cpu().numpy()
            lr["k_in"] = lb["k_in"][:rows].float().cpu().numpy()
            lr["v_in"] = lb["v_in"][:rows].float().cpu().numpy()
            rec["layers"].append(lr)
        G.append(rec)
    return G


def oracle_block(inp, w, sched, G):
    """The block oracle on the same inputs, in lock step with the GPU run G
    (its statistics and pre-quantisation K/V of quantised levels);
    sched["rho"] must reproduce G's counts."""
    ov = {}
    L = len(inp["layers"])
    for r in range(2, len(G) + 1):
        ov[("stat", r)] = G[r - 1]["stat"]
        for l in range(L):
            if "cstat" in G[r - 2]["layers"][l]:
                ov[("cstat", r, l)] = G[r - 2]["layers"][l]["cstat"]
    for r in range(1, len(G) + 1):
        if sched["bits"][r - 1] == 32:
            continue            # raw levels: no quantisation decision to align
        for l in range(L):
            gl = G[r - 1]["layers"][l]
            ov[("kvin", r, l)] = dict(k=gl["k_in"], v=gl["v_in"])
    layers = [{k: synth.bf16_bits_to_f32(v) for k, v in lw.items()} for lw in inp["layers"]]
    s = dict(sched)
    s["R"] = len(G)
    return ob.run_block(inp["h1"], layers, s, theta=w.extra["theta"], eps=w.extra["eps"],
                        override=ov, bf16_acts=True)


def check_codes_exact(gl, ol, bits, d, asym, tag):
    """The GPU's stored level (codes, scales, offsets) against the oracle's
    quantisation of the same pre-quantisation values, bit for bit."""
    lk, lv = ol["level_k"], ol["level_v"]
    for kv, lev in (("k", lk), ("v", lv)):
        mine = ob.unpack_codes(gl["kv"][kv], bits, d, unsigned=asym)
        np.testing.assert_array_equal(mine, lev["codes"].astype(np.int16), err_msg=f"{tag} {kv} codes")
        np.testing.assert_array_equal(gl["kv"][kv + "s"].view(np.uint32),
                                      np.asarray(lev["scales"], np.float32).view(np.uint32),
                                      err_msg=f"{tag} {kv} scales")
        if asym:
            np.testing.assert_array_equal(gl["kv"][kv + "z"].view(np.uint32),
                                          np.asarray(lev["zeros"], np.float32).view(np.uint32),
                                          err_msg=f"{tag} {kv} offsets")
