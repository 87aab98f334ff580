"""Pins of the generation oracle (oracle/decode.py: run_generation,
append_token, append_block) against closed forms in float64 numpy, exact
bookkeeping and the prompt's own quantisation:

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
  the window's columns in the cached mass bookkeeping (Sec. 4.2);
* under the paper's quantiser (App. E) tokens leave the window g at a time;
  an appended block is quantised exactly as the same tokens would be at the
  end of a prompt whose length is a multiple of g (every token active), and,
  after a prompt of any length, exactly as a prompt of those g tokens alone
  (a key group of its own)."""
import numpy as np

from oracle import decode as od
from sparse_attention_kv_amd import synth


def _sched(N=120, H=2, d=64, R=3, kcols=(120, 40, 20), rho=(1.0, 0.5, 0.25), bits=(8, 4, 2),
           quant="absmax"):
    return dict(N=N, H=H, d=d, g=32, R=R, n_sink=4, rho=list(rho), kcols=list(kcols),
                bits=list(bits), quant=quant)


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
                Kc[r] = np.concatenate([Kc[r], rec["appended"][0][r]["khat"][None]])
                Vc[r] = np.concatenate([Vc[r], rec["appended"][0][r]["vhat"][None]])
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


def test_asym_window_leaves_in_blocks_of_g():
    sc = _sched(kcols=(120, 120, 120), bits=(4, 4, 4), quant="asym")
    g, W = sc["g"], 3
    k, v, stat, gq, gk, gv = _inputs(sc, W + 2 * g + 2)
    cache = od.build_cache(k, v, stat, sc)
    res = od.run_generation(cache, gq, gk, gv, sc, window=W)
    for t, rec in enumerate(res):
        f = g * max(0, (t - W) // g)      # tokens appended before token t
        assert rec["N"] == sc["N"] + f
        assert rec["T"] == t - f + 1 and W + 1 <= rec["T"] + (g if t < W + g else 0)
        made = rec["appended"] is not None
        assert made == (t >= W + g and (t - W) % g == 0)
        if made:
            assert len(rec["appended"]) == 1
            assert rec["appended"][0][0]["k_codes"].shape == (g, sc["H"], sc["d"])


def _all_active(sc, N):
    return dict(sc, N=N, rho=[1.0] * sc["R"], kcols=[N] * sc["R"])


def test_asym_block_matches_prompt_quantisation():
    # every token active at every loop and a prompt of 3 whole groups: the
    # block is the 4th group of a prompt of N + g tokens, bit for bit
    for bits in ((4, 4, 4), (8, 4, 2)):
        sc = _all_active(_sched(bits=bits, quant="asym"), 96)
        g, N = sc["g"], 96
        k, v, stat, _, gk, gv = _inputs(sc, g)
        app = od.append_block(gk, gv, sc)
        kl = [np.concatenate([k[r], np.stack([t[r] for t in gk])]) for r in range(sc["R"])]
        vl = [np.concatenate([v[r], np.stack([t[r] for t in gv])]) for r in range(sc["R"])]
        st = [None] + [np.arange(N + g, dtype=np.float32)] * (sc["R"] - 1)
        full = od.build_cache(kl, vl, st, dict(sc, N=N + g, kcols=[N + g] * sc["R"]))
        for r in range(sc["R"]):
            np.testing.assert_array_equal(app[r]["khat"], full[r]["khat"][N:])
            np.testing.assert_array_equal(app[r]["vhat"], full[r]["vhat"][N:])
            np.testing.assert_array_equal(app[r]["k_codes"], full[r]["k_codes"][N:])
            np.testing.assert_array_equal(app[r]["k_scale"], full[r]["k_scale"][N // g:])
            np.testing.assert_array_equal(app[r]["v_zero"], full[r]["v_zero"][N:])


def test_asym_block_is_a_group_of_its_own():
    # after a prompt of 120 tokens (a partial last group) the block is
    # quantised as a g-token prompt by itself
    sc = _sched(bits=(4, 2, 2), quant="asym")
    g = sc["g"]
    _, _, _, _, gk, gv = _inputs(sc, g, seed=9)
    app = od.append_block(gk, gv, sc)
    alone = od.build_cache([np.stack([t[r] for t in gk]) for r in range(sc["R"])],
                           [np.stack([t[r] for t in gv]) for r in range(sc["R"])],
                           [None] + [np.zeros(g, np.float32)] * (sc["R"] - 1),
                           _all_active(sc, g))
    for r in range(sc["R"]):
        np.testing.assert_array_equal(app[r]["khat"], alone[r]["khat"])
        np.testing.assert_array_equal(app[r]["k_zero"], alone[r]["k_zero"])
        np.testing.assert_array_equal(app[r]["v_codes"], alone[r]["v_codes"])
        # one key group: a channel's codes span the full range of its levels
        assert app[r]["k_scale"].shape == (1, sc["H"], sc["d"])


def test_asym_unpruned_generation_is_dense_softmax():
    sc = _sched(kcols=(120, 1000, 1000), bits=(4, 4, 4), quant="asym")
    g, W = sc["g"], 2
    k, v, stat, gq, gk, gv = _inputs(sc, W + g + 3)
    cache = od.build_cache(k, v, stat, sc)
    res = od.run_generation(cache, gq, gk, gv, sc, window=W)
    sm = 1.0 / np.sqrt(sc["d"])
    Kc = [cache[r]["khat"] for r in range(sc["R"])]
    Vc = [cache[r]["vhat"] for r in range(sc["R"])]
    f = 0
    for t, rec in enumerate(res):
        for blk in rec["appended"] or []:
            for r in range(sc["R"]):
                Kc[r] = np.concatenate([Kc[r], blk[r]["khat"]])
                Vc[r] = np.concatenate([Vc[r], blk[r]["vhat"]])
            f += g
        assert rec["N"] == Kc[0].shape[0]
        for r, lrec in enumerate(rec["recs"], start=1):
            K = np.concatenate([Kc[r - 1], np.stack([gk[u][r - 1] for u in range(f, t + 1)])])
            V = np.concatenate([Vc[r - 1], np.stack([gv[u][r - 1] for u in range(f, t + 1)])])
            o, lse = _dense64(gq[t][r - 1], K, V, sm)
            np.testing.assert_allclose(lrec["out"], o, rtol=0, atol=2e-5)
            np.testing.assert_allclose(lrec["lse"], lse, rtol=0, atol=2e-5)
    assert f == g
