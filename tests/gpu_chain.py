"""Helpers for the GPU parity tests: run the whole R-loop step through the
C ABI (``fl_loop_step``) and read back every loop's results, then run the
oracle on the same inputs, feeding it the GPU's own fp32 statistic buffers
for its selections (index sets are then unique and compared exactly)."""
import numpy as np
import torch

import oracle
from oracle.loop import run_prefill
from sparse_attention_kv_amd import fl, synth


def to_dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def counts(w):
    n = [w.N]
    for r in range(1, w.R):
        n.append(oracle.active_count(w.rho[r], w.N, n[-1]))
    return n


def run_gpu(w, inp, mode=fl.FL_DEQ_AUTO, bits=None, token_stat=fl.FL_TOKEN_STAT_ABS,
            col_stat=fl.FL_COL_STAT_MASS, quant=fl.FL_QUANT_ABSMAX):
    bits = bits or w.bits
    dt = inp["dtype"]
    dev = {key: [to_dev(a, dt) for a in inp[key]] for key in ("h", "q", "k", "v")}
    n_act = counts(w)
    runner = fl.LoopRunner(w.N, w.H, w.d, w.g, w.R, w.n_sink, n_act, w.kcols, bits,
                           dtype=torch.bfloat16 if dt == "bf16" else torch.float32, mode=mode,
                           token_stat=token_stat, col_stat=col_stat, quant=quant)
    res = []
    for r in range(1, w.R + 1):
        hp = dev["h"][r - 2] if r > 1 else None
        qp = dev["q"][r - 2] if r > 1 else None
        runner.step(r, dev["h"][r - 1], hp, dev["q"][r - 1], dev["k"][r - 1], dev["v"][r - 1], qp)
        torch.cuda.synchronize()
        rec = dict(r=r)
        act = runner.active[r - 1].cpu().numpy()
        rec["active"] = act
        if r > 1:
            rec["stat"] = runner.stat[: n_act[r - 2]].cpu().numpy().copy()
            rec["slot"] = runner.slot[r - 1].cpu().numpy()
        cb = runner.codes[r - 1]
        rec["k_codes"] = cb["k"].cpu().numpy()
        rec["v_codes"] = cb["v"].cpu().numpy()
        rec["k_scale"] = cb["ks"].cpu().numpy()
        rec["v_scale"] = cb["vs"].cpu().numpy()
        if "kz" in cb:
            rec["k_zero"] = cb["kz"].cpu().numpy()
            rec["v_zero"] = cb["vz"].cpu().numpy()
        sel = runner.sel_used(r)
        rec["sel"] = None if sel is None else sel.cpu().numpy()
        rec["k"] = runner.k_used(r)
        need_c = r < w.R and w.kcols[r] < rec["k"]
        rec["cstat"] = runner.col_stat[r - 1][:, : rec["k"]].cpu().numpy().copy() if need_c else None
        rec["out"] = runner.out.cpu().numpy()[act]
        rec["lse"] = runner.lse.cpu().numpy()[act]
        rec["mass_u"] = runner.mass_u.cpu().numpy()[act]
        rec["out_u"] = runner.out_u.cpu().numpy()[act]
        res.append(rec)
    return res, runner


def oracle_stat_names(token_stat, col_stat):
    return dict(token_stat="rel" if token_stat == fl.FL_TOKEN_STAT_REL else "abs",
                col_stat="vnorm" if col_stat == fl.FL_COL_STAT_VNORM else "mass")


def run_oracle_lockstep(w, inp, gres, bits=None, token_stat=fl.FL_TOKEN_STAT_ABS,
                        col_stat=fl.FL_COL_STAT_MASS, quant=fl.FL_QUANT_ABSMAX):
    x = synth.as_f32_inputs(inp)
    sched = w.sched()
    sched.update(oracle_stat_names(token_stat, col_stat))
    if quant == fl.FL_QUANT_ASYM:
        sched["quant"] = "asym"
    if bits:
        sched["bits"] = list(bits)
    ov = {}
    for r in range(2, w.R + 1):
        ov[("stat", r)] = gres[r - 1]["stat"]
        if gres[r - 2]["cstat"] is not None:
            ov[("cstat", r)] = gres[r - 2]["cstat"]
    return run_prefill(x["h"], x["q"], x["k"], x["v"], sched, override=ov)


def rel_l2(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def assert_close(got, want, what, rel=1e-2, mabs=3e-2, ref_norm=None):
    """rel-L2 (against ref_norm when given) and max-abs bounds."""
    got = np.asarray(got, np.float64); want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if ref_norm is None:
        e = rel_l2(got, want)
    else:
        e = float(np.linalg.norm(got - want) / max(ref_norm, 1e-30))
    m = float(np.max(np.abs(got - want))) if got.size else 0.0
    if not (e <= rel and m <= mabs):
        idx = np.unravel_index(np.argmax(np.abs(got - want)), got.shape)
        print(f"  {what}: worst at {idx}: got {got[idx]:.5f} want {want[idx]:.5f}; "
              f"max |want| {np.abs(want).max():.3f}", flush=True)
    assert e <= rel and m <= mabs, f"{what}: rel-L2 {e:.3e} (<= {rel}), max-abs {m:.3e} (<= {mabs})"
    return e, m


def assert_close_scaled(got, want, what, rel=1e-2, mabs=3e-2):
    """Column statistics are sums of up to N probabilities (values up to
    ~N at sink columns): rel-L2 <= rel and |got - want| <= mabs * max(1, |want|)
    elementwise (the absolute bound in units of one row's probability mass)."""
    got = np.asarray(got, np.float64); want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    e = rel_l2(got, want)
    lim = mabs * np.maximum(1.0, np.abs(want))
    worst = float(np.max(np.abs(got - want) / lim)) if got.size else 0.0
    assert e <= rel and worst <= 1.0, f"{what}: rel-L2 {e:.3e} (<= {rel}), scaled max {worst:.3f} (<= 1)"
    return e, worst


def assert_close_bf16(got, want, what, rel=1e-2, mabs=3e-2):
    """Activations of the looped block stored as bf16 by two implementations
    (keys and values before quantisation: a bf16 projection of the RMSNorm'd
    hidden state, RoPE, a second bf16 rounding), rows [n][...] per token.
    Two parts make their difference:
      * bf16 keeps 8 significant bits, so values summed in different orders
        round to neighbours one ulp (2^-8 to 2^-7 of the value) apart at each
        rounding -- a value in [4, 8) already has an ulp of 2^-5 > 3e-2;
      * the hidden state's own difference (bounded in units of its row's
        RMS, see assert_close_state), carried through RMSNorm and the
        projection, is spread over the whole row of the token.
    Elementwise |got - want| <= mabs * max(1, |want|, rms(want row)) (about
    four ulps of the value, or 3e-2 of the row's scale), rel-L2 <= rel."""
    got = np.asarray(got, np.float64); want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    e = rel_l2(got, want)
    w2 = want.reshape(want.shape[0], -1)
    rms = np.sqrt(np.mean(w2 * w2, axis=1)).reshape((-1,) + (1,) * (want.ndim - 1))
    lim = mabs * np.maximum(np.maximum(1.0, np.abs(want)), rms)
    worst = float(np.max(np.abs(got - want) / lim)) if got.size else 0.0
    if not (e <= rel and worst <= 1.0):
        idx = np.unravel_index(np.argmax(np.abs(got - want) / lim), got.shape)
        print(f"  {what}: worst at {idx}: got {got[idx]:.5f} want {want[idx]:.5f}", flush=True)
    assert e <= rel and worst <= 1.0, f"{what}: rel-L2 {e:.3e} (<= {rel}), scaled max {worst:.3f} (<= 1)"
    return e, worst


def assert_close_state(got, want, what, rel=1e-2, mabs=3e-2):
    """The looped block's fp32 residual stream h [N][D].  Its bounds follow
    from how the block reads it: every layer sees h only through RMSNorm,
    i.e. relative to each row's RMS, so an elementwise difference counts in
    units of its row's RMS: |got - want| <= mabs * max(1, rms(want row)),
    with rel-L2 <= rel over the whole state.  (An attention output that
    differs within the attention bound moves every later row of h through
    the output projection, and rows updated in more loops carry larger
    states and larger absolute differences.)"""
    got = np.asarray(got, np.float64); want = np.asarray(want, np.float64)
    assert got.shape == want.shape and got.ndim == 2, (what, got.shape, want.shape)
    e = rel_l2(got, want)
    rms = np.sqrt(np.mean(want * want, axis=1, keepdims=True))
    lim = mabs * np.maximum(1.0, rms)
    ratio = np.abs(got - want) / lim
    worst = float(ratio.max()) if got.size else 0.0
    m = float(np.max(np.abs(got - want))) if got.size else 0.0
    if not (e <= rel and worst <= 1.0):
        idx = np.unravel_index(np.argmax(ratio), got.shape)
        print(f"  {what}: worst at {idx}: got {got[idx]:.5f} want {want[idx]:.5f} "
              f"(row rms {rms[idx[0], 0]:.3f})", flush=True)
    assert e <= rel and worst <= 1.0, (f"{what}: rel-L2 {e:.3e} (<= {rel}), max-abs {m:.3e}, "
                                       f"row-scaled max {worst:.3f} (<= 1)")
    return e, m, worst


def compare_chain(w, gres, ores, bits=None, check_codes=True, quant=fl.FL_QUANT_ABSMAX):
    bits = bits or w.bits
    report = []
    for r in range(1, w.R + 1):
        g, o = gres[r - 1], ores[r - 1]
        np.testing.assert_array_equal(g["active"], o["active"], err_msg=f"loop {r} active set")
        if r > 1:
            np.testing.assert_allclose(g["stat"], o["stat"], rtol=1e-5, err_msg=f"loop {r} stat")
            slot = np.full(w.N, -1, np.int32)
            slot[o["active"]] = np.arange(len(o["active"]))
            np.testing.assert_array_equal(g["slot"], slot, err_msg=f"loop {r} slot map")
        if check_codes:
            for kv in ("k", "v"):
                lvl = o["level_" + kv]
                if quant == fl.FL_QUANT_ASYM:
                    np.testing.assert_array_equal(g[kv + "_codes"],
                                                  oracle.pack_codes(lvl["codes"], bits[r - 1]),
                                                  err_msg=f"loop {r} {kv} codes")
                    for part, key in (("_scale", "scales"), ("_zero", "zeros")):
                        np.testing.assert_array_equal(g[kv + part].view(np.uint32),
                                                      lvl[key].view(np.uint32),
                                                      err_msg=f"loop {r} {kv}{part}")
                elif bits[r - 1] == 32:
                    raw = g[kv + "_codes"].view(np.float32).reshape(lvl["raw"].shape)
                    np.testing.assert_array_equal(raw, lvl["raw"], err_msg=f"loop {r} raw {kv}")
                else:
                    packed = oracle.pack_codes(lvl["codes"], bits[r - 1])
                    np.testing.assert_array_equal(g[kv + "_codes"], packed,
                                                  err_msg=f"loop {r} {kv} codes")
                    np.testing.assert_array_equal(g[kv + "_scale"].view(np.uint32),
                                                  lvl["scales"].view(np.uint32),
                                                  err_msg=f"loop {r} {kv} scales")
        if o["sel"] is None:
            assert g["sel"] is None and g["k"] == w.N
        else:
            np.testing.assert_array_equal(g["sel"], o["sel"], err_msg=f"loop {r} columns")
        e_o = assert_close(g["out"], o["out"], f"loop {r} out")
        e_l = assert_close(g["lse"], o["lse"], f"loop {r} lse")
        assert_close(g["mass_u"], o["mass_u"], f"loop {r} mass_u", mabs=3e-2)
        if o["out_u"] is not None:
            # O_U adds straight into the output: bounded like the output
            # (max-abs, and L2 error relative to the output's norm)
            assert_close(g["out_u"], o["out_u"], f"loop {r} out_u",
                         ref_norm=float(np.linalg.norm(o["out"])))
            # and relative to its own norm: the subtract form o_prev - sum_S P V
            # loses digits when O_U is a small share of the output, so the
            # bound is 5 %, or 3e-3 of the output's norm where O_U is smaller
            # (measured: median 1 %, at most 8 % where |O_U| = 1.5 % of |out|)
            own = rel_l2(g["out_u"], o["out_u"])
            share = np.linalg.norm(o["out_u"]) / max(np.linalg.norm(o["out"]), 1e-30)
            assert own <= max(5e-2, 3e-3 / max(share, 1e-30)), \
                f"loop {r} out_u: rel-L2 to its own norm {own:.3e} at |O_U|/|out| = {share:.3e}"
        if o["cstat"] is not None:
            assert g["cstat"] is not None
            assert_close_scaled(g["cstat"], o["cstat"], f"loop {r} cstat")
        report.append((r, e_o, e_l))
    return report
