"""Helpers of the batched-decode GPU tests: fill B sequences' caches and run
the R loops of their new tokens through the C ABI (``fl_decode_step``), then
run the decode oracle for chosen sequences, feeding it the GPU's column
statistics for its column selections (index sets then compared exactly)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from oracle import decode as od
from sparse_attention_kv_amd import fl, synth

from gpu_chain import assert_close, assert_close_scaled, counts, to_dev


def _draw(w, B, threads):
    """Yields (b, inputs) in order, at most `threads` sequences in flight."""
    with ThreadPoolExecutor(threads) as ex:
        for b0 in range(0, B, threads):
            futs = [ex.submit(synth.gen_decode_seq, w, b) for b in range(b0, min(B, b0 + threads))]
            for i, f in enumerate(futs):
                yield b0 + i, f.result()


def _quant(w):
    return fl.FL_QUANT_ASYM if w.extra.get("quant") == "asym" else fl.FL_QUANT_ABSMAX


def _sched(w):
    sched = w.sched()
    if w.extra.get("quant") == "asym":
        sched["quant"] = "asym"
    return sched


def run_decode_gpu(w, keep=(), threads=8):
    B, N, H, d, R = w.extra["B"], w.N, w.H, w.d, w.R
    n_act = counts(w)
    run = fl.DecodeRunner(B, N, H, d, w.g, R, w.n_sink, n_act, w.kcols, w.bits, quant=_quant(w))
    tok = {key: np.empty((R, B, H, d), np.uint16) for key in ("q_new", "k_new", "v_new")}
    kept = {}
    for b, x in _draw(w, B, threads):
        k = [to_dev(a, "bf16") for a in x["k"]]
        v = [to_dev(a, "bf16") for a in x["v"]]
        st = [None] + [torch.from_numpy(s).cuda() for s in x["stat"][1:]]
        run.load_sequence(b, k, v, st)
        for key in tok:
            for r in range(R):
                tok[key][r, b] = x[key][r]
        if b in keep:
            kept[b] = x
        del k, v, st
    torch.cuda.synchronize()
    dev = {key: [to_dev(tok[key][r], "bf16") for r in range(R)] for key in tok}
    res = []
    for r in range(1, R + 1):
        prev = [dev[key][r - 2] if r > 1 else None for key in ("q_new", "k_new", "v_new")]
        run.step(r, dev["q_new"][r - 1], dev["k_new"][r - 1], dev["v_new"][r - 1], *prev)
        torch.cuda.synchronize()
        kk = run.k_used(r)
        sel = run.sel_used(r)
        need_c = r < R and w.kcols[r] < kk
        res.append(dict(r=r, k=kk, sel=None if sel is None else sel.cpu().numpy(),
                        out=run.out.cpu().numpy(), lse=run.lse.cpu().numpy(),
                        mass_u=run.mass_u.cpu().numpy(), out_u=run.out_u.cpu().numpy(),
                        cstat=run.col_stat[r - 1][:, :, :kk].cpu().numpy() if need_c else None))
        print(f"  gpu decode loop {r}: k={kk}", flush=True)
    return res, kept, run


def check_sequence(w, b, x, gres, run):
    """Cache levels of sequence b bit-exact, then every loop's results."""
    sched = _sched(w)
    asym = sched.get("quant") == "asym"
    f = synth.bf16_bits_to_f32
    cache = od.build_cache([f(a) for a in x["k"]], [f(a) for a in x["v"]], x["stat"], sched)
    for r in range(1, w.R + 1):
        lv = cache[r - 1]
        if r > 1:
            np.testing.assert_array_equal(run.rows[r - 1][b].cpu().numpy(), lv["active"],
                                          err_msg=f"seq {b} loop {r} active set")
        cb = run.codes[r - 1]
        for kv in ("k", "v"):
            np.testing.assert_array_equal(cb[kv][b].cpu().numpy(),
                                          oracle.pack_codes(lv[kv + "_codes"], w.bits[r - 1]),
                                          err_msg=f"seq {b} loop {r} {kv} codes")
            np.testing.assert_array_equal(cb[kv + "s"][b].cpu().numpy().view(np.uint32),
                                          lv[kv + "_scale"].view(np.uint32),
                                          err_msg=f"seq {b} loop {r} {kv} scales")
            if asym:
                np.testing.assert_array_equal(cb[kv + "z"][b].cpu().numpy().view(np.uint32),
                                              lv[kv + "_zero"].view(np.uint32),
                                              err_msg=f"seq {b} loop {r} {kv} zeros")
    ov = {("cstat", r): gres[r - 2]["cstat"][b] for r in range(2, w.R + 1)
          if gres[r - 2]["cstat"] is not None}
    recs = od.run_decode(cache, [f(a) for a in x["q_new"]], [f(a) for a in x["k_new"]],
                         [f(a) for a in x["v_new"]], sched, override=ov)
    errs = []
    for r in range(1, w.R + 1):
        g, o = gres[r - 1], recs[r - 1]
        assert g["k"] == o["k"], (b, r, g["k"], o["k"])
        if o["sel"] is None:
            assert g["sel"] is None
        else:
            np.testing.assert_array_equal(g["sel"][b], o["sel"], err_msg=f"seq {b} loop {r} columns")
        e = assert_close(g["out"][b], o["out"], f"seq {b} loop {r} out")
        assert_close(g["lse"][b], o["lse"], f"seq {b} loop {r} lse")
        assert_close(g["mass_u"][b], o["mass_u"], f"seq {b} loop {r} mass_u")
        assert_close(g["out_u"][b], o["out_u"], f"seq {b} loop {r} out_u",
                     ref_norm=float(np.linalg.norm(o["out"])))
        if o["cstat"] is not None:
            assert g["cstat"] is not None
            assert_close_scaled(g["cstat"][b], o["cstat"], f"seq {b} loop {r} cstat")
        errs.append(e)
    return errs
