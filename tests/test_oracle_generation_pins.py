"""Pins of the generation oracle (oracle/decode.py: run_generation,
append_token) against closed forms in float64 numpy and exact bookkeeping:

* window bookkeeping (App. E keeps the most recent tokens in BF16): token t
  attends to N0 + max(0, t - W) cached positions and min(t, W) + 1
  unquantised columns, the cache growing one position per token once the
  window is full, in token order;
* an appended token's cache rows are its own residual chain: codes x scales
  summed level by level in fp32 give the returned dequantised values bit for
  bit, and raw levels reproduce its inputs exactly;
* with unpruned budgets every loop of every generated token is plain softmax
  attention over the grown cache plus the window (Sec. 4.2 with all columns);
* frozen loops (unchanged inputs, raw levels) restore loop 1's output with
  the window's columns in the cached mass bookkeeping (Sec. 4.2)."""
import numpy as np

from oracle import decode as od
from sparse_attention_kv_amd import synth


def _sched(N=120, H=2, d=64, R=3, kcols=(120, 40, 20), rho=(1.0, 0.5, 0.25), bits=(8, 4, 2)):
    return dict(N=N, H=H, d=d, g=32, R=R, n_sink=4, rho=list(rho), kcols=list(kcols),
                bits=list(bits))


def _inputs(sc, n_gen, seed=7, frozen=False):
    w = synth.WORKLOADS["decode64x8k"].scaled(N=sc["N"], H=sc["H"], d=sc["d"], R=sc["R"],
                                              g=sc["g"], rho=sc["rho"], kcols=sc["kcols"],
                                              bits=sc["bits"], seed=seed)
    w.extra = dict(B=1)
    x = synth.gen_decode_seq(w, 0, n_gen=n_gen)
    f = synth.bf16_bits_to_f32
    k = [f(a) for a in x["k"]]; v = [f(a) for a in x["v"]]
    gq = [[f(a) for a in t] for t in x["gen_q"]]
    gk = [[f(a) for a in t] for t in x["gen_k"]]
    gv = [[f(a) for a in t] for t in x["gen_v"]]
    if frozen:
        k = [k[0]] * sc["R"]; v = [v[0]] * sc["R"]
        gq = [[t[0]] * sc["R"] for t in gq]; gk = [[t[0]] * sc["R"] for t in gk]
        gv = [[t[0]] * sc["R"] for t in gv]
    return k, v, x["stat"], gq, gk, gv


def _dense64(q, K, V, sm):
    s = np.einsum("hd,nhd->hn", q.astype(np.float64), K.astype(np.float64)) * float(sm)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return np.einsum("hn,nhd->hd", e / z, V.astype(np.float64)), (m + np.log(z))[:, 0]


def test_window_bookkeeping():
    sc = _sched(kcols=(120, 120, 120))
    k, v, stat, gq, gk, gv = _inputs(sc, 9)
    cache = od.build_cache(k, v, stat, sc)
    W = 3
    res = od.run_generation(cache, gq, gk, gv, sc, window=W)
    for t, rec in enumerate(res):
        assert rec["N"] == sc["N"] + max(0, t - W)
        assert rec["T"] == min(t, W) + 1
        assert (rec["appended"] is None) == (t < W + 1)


def test_appended_rows_are_the_tokens_chain():
    for bits in ((8, 4, 2), (8, 32, 32)):
        sc = _sched(bits=bits)
        _, _, _, _, gk, gv = _inputs(sc, 1)
        app = od.append_token(gk[0], gv[0], sc)
        g = sc["g"]
        x = np.zeros((sc["H"], sc["d"]), np.float32)
        for r, lv in enumerate(app, start=1):
            if bits[r - 1] == 32:
                # raw level: the chain reproduces the input exactly
                np.testing.assert_array_equal(lv["khat"], gk[0][r - 1])
                x = lv["khat"]
                continue
            term = (lv["k_codes"][0].astype(np.float32) *
                    np.repeat(lv["k_scale"][0], g, axis=-1)).astype(np.float32)
            x = term if r == 1 else (x + term).astype(np.float32)
            np.testing.assert_array_equal(lv["khat"], x)


def test_unpruned_generation_is_dense_softmax():
    # budgets above the grown context (120 prompt + up to 5 appended tokens)
    sc = _sched(kcols=(120, 1000, 1000))
    k, v, stat, gq, gk, gv = _inputs(sc, 8)
    cache = od.build_cache(k, v, stat, sc)
    W = 3
    res = od.run_generation(cache, gq, gk, gv, sc, window=W)
    sm = 1.0 / np.sqrt(sc["d"])
    Kc = [cache[r]["khat"] for r in range(sc["R"])]
    Vc = [cache[r]["vhat"] for r in range(sc["R"])]
    for t, rec in enumerate(res):
        if rec["appended"] is not None:
            for r in range(sc["R"]):
                Kc[r] = np.concatenate([Kc[r], rec["appended"][r]["khat"][None]])
                Vc[r] = np.concatenate([Vc[r], rec["appended"][r]["vhat"][None]])
        lo = max(0, t - W)
        for r, lrec in enumerate(rec["recs"], start=1):
            K = np.concatenate([Kc[r - 1], np.stack([gk[u][r - 1] for u in range(lo, t + 1)])])
            V = np.concatenate([Vc[r - 1], np.stack([gv[u][r - 1] for u in range(lo, t + 1)])])
            o, lse = _dense64(gq[t][r - 1], K, V, sm)
            np.testing.assert_allclose(lrec["out"], o, rtol=0, atol=2e-5)
            np.testing.assert_allclose(lrec["lse"], lse, rtol=0, atol=2e-5)


def test_frozen_generation_restores_dense_output():
    sc = _sched(bits=(32, 32, 32))
    k, v, stat, gq, gk, gv = _inputs(sc, 6, frozen=True)
    cache = od.build_cache(k, v, stat, sc)
    res = od.run_generation(cache, gq, gk, gv, sc, window=2)
    for rec in res:
        recs = rec["recs"]
        for r in (2, 3):
            assert recs[r - 1]["sel"] is not None
            np.testing.assert_allclose(recs[r - 1]["out"], recs[0]["out"], rtol=0, atol=3e-5)
