#!/usr/bin/env python
"""Benchmark of FlashLoop's lazy-update loop attention step on one MI355X.

A step is one full pass of the R-loop attention step over one synthetic
sequence: loop 1 (int8 base quantisation, dense causal attention, column
statistics) then loops 2..R (token statistic + nested top-k, residual
quantisation, column selection, cache rebuild when the column set shrinks,
sparse attention, column statistics when the next loop prunes).  Inputs are
resident in HBM before the timed region.

value = active-query tokens per second of the sparse loops' attention step:
        sum_{r=2..R} n_r over the time of steps a5-a8 (column selection,
        pruned-column caches, sparse attention, column statistics) of loops
        2..R.  Steps a1-a4 of those loops and the dense first loop are
        reported beside it, and ms_per_step is the whole step.

Prints ONE JSON line.  Extra fields: per-loop and per-phase times, per-kernel
times, the roofline of the dominant kernel of the metric's work and of that
work as a whole (algorithmic flops from the actual index sets), loop 1's
dense attention roofline, KV bytes/token, and the CPU oracle timed on a
bounded sample of the same work.  The default prefill line also carries the
batched-decode workload (64 x 8K) under "decode64x8k" and the 24-layer
looped block (8K) under "block8k" (--no-decode / --no-block skip them).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "active-query tokens/s of loop-r sparse attention @32K, R=4; KV bytes/token; %roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# library timing names -> kernel symbols as rocprofv3 reports them (d = 128)
KERNEL_SYMBOL = {"attn": "k_attn_lds<128, 0, 0, 64>", "attn_split": "k_attn_lds<128, 0, 1, 32>",
                 "attn_ad": "k_attn_ad<128, 0>", "attn_ad_rebuild": "k_attn_ad<128, 1>",
                 "attn_ad_rebuild_add": "k_attn_ad<128, 2>", "attn_ad_rb": "k_attn_ad<128, 3>",
                 "attn_rebuild": "k_attn_lds<128, 1, 0, 64>", "colstat": "k_colstat_lds<128, 0, 4, 2>",
                 "colstat_split": "k_colstat_lds<128, 1, 4, 1>", "decode_dense": "k_decode<128, 0, false, true, false, 0>",
                 "decode": "k_decode<128, 0, true, false, false, 0>",
                 "decode_rebuild": "k_decode<128, 1, true, true, false, 0>"}
# projections of the 2048-hidden block: epilogue (0 store, 1 residual, 2 SwiGLU)
# and tile width; o and down share one instantiation, so only the others are
# separable in a trace
BLOCK_GEMM_SYMBOL = {"gemm_qkv": "k_gemm_lds<0, 128>", "gemm_gate_up": "k_gemm_lds<2, 128>"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill32k")
    ap.add_argument("--cpu-rows", type=int, default=1536,
                    help="query rows per loop in the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="prefill32k: skip the batched-decode measurement attached to the line")
    ap.add_argument("--no-block", action="store_true",
                    help="prefill32k: skip the 24-layer block measurement attached to the line")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    ap.add_argument("--token-stat", default="abs", choices=["abs", "rel"],
                    help="token ranking: absolute or normalised hidden-state change")
    ap.add_argument("--col-stat", default="mass", choices=["mass", "vnorm"],
                    help="column ranking: probability mass, or mass x value norm")
    ap.add_argument("--quant", default="absmax", choices=["absmax", "asym"],
                    help="cache quantiser: absmax int8 base + int4/int2 residuals, or the "
                         "paper's asymmetric INT4 (keys per channel, values per token)")
    ap.add_argument("--quant-study", action="store_true",
                    help="residual vs direct quantisation error by loop on the prefill inputs")
    ap.add_argument("--sweep", default=None, choices=["length", "depth"],
                    help="context-length (4K-32K) or depth (R = 4..32) sweep of the step")
    ap.add_argument("--generate", action="store_true",
                    help="decode workloads: generation with a bf16 window and cache appends")
    ap.add_argument("--gen-warmup", type=int, default=16)
    ap.add_argument("--gen-timed", type=int, default=16)
    ap.add_argument("--calibrate", action="store_true",
                    help="block workloads: time the retention calibration instead of the step")
    ap.add_argument("--mode", default="auto", choices=["auto", "once", "in_tile"],
                    help="where the cache is dequantised (library default: auto)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_traffic(workload, kernel):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3 PMC
    summary (FETCH_SIZE / WRITE_SIZE scaled by a reference copy), or None
    when there is none or the kernel's sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        f = line.rstrip("\n").split("\t")
        if f[0] != kernel:
            continue
        src, digest = f[1].split(":")
        h = hashlib.sha256()
        for p in (src, "fl_device.h", "fl_kernels.h"):
            with open(os.path.join(ROOT, "sparse_attention_kv_amd", "csrc", p), "rb") as fh:
                h.update(fh.read())
        return int(f[5]) if h.hexdigest()[:16] == digest else None
    return None


def pairs_per_head(torch, act, sel, N):
    """sum over heads and active rows of |S(i)| = #selected columns <= i."""
    a = act.to(torch.int64)
    if sel is None:
        return int((a + 1).sum().item()), None
    cnt = torch.searchsorted(sel.to(torch.int64).contiguous(), a.expand(sel.shape[0], -1).contiguous(),
                             right=True)
    return int(cnt.sum().item()) // 1, cnt


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_attention_kv_amd import fl, synth

    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] reference copy of {args.calib_copy_mib} MiB done")
    if args.quant == "asym":
        w = w.scaled(bits=[4] * w.R)          # the paper's INT4 base and residuals
    if args.quant_study:
        return bench_quant_study(args, w, np, torch, fl, synth)
    if w.kind == "block":
        return bench_block(args, w, np, torch, fl, synth)
    if w.kind == "decode":
        if args.generate:
            return bench_generate(args, w, np, torch, fl, synth)
        print(json.dumps(bench_decode(args, w, np, torch, fl, synth)), flush=True)
        return
    if args.sweep:
        return bench_sweep(args, w, np, torch, fl, synth)
    out = bench_prefill(args, w, np, torch, fl, synth, cpu=not args.no_cpu_baseline)
    if w.name == "prefill32k" and not args.no_decode and args.quant == "absmax":
        out["decode64x8k"] = decode_summary(args, np, torch, fl, synth)
    if w.name == "prefill32k" and not args.no_block and args.quant == "absmax":
        out["block8k"] = block_summary(args, np, torch, fl, synth)
    print(json.dumps(out), flush=True)


def block_summary(args, np, torch, fl, synth):
    """The 24-layer looped block (8K tokens, R=4, token-sparse projections,
    sparse loop attention, residual KV store) timed after the prefill and
    decode measurements, 5 steps after 2 warm-up steps, no CPU baseline: its
    active tokens/s, per-loop times and the gate/up projection's roofline."""
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    bargs = argparse.Namespace(**vars(args))
    bargs.steps, bargs.warmup, bargs.no_cpu_baseline = 5, 2, True
    bargs.calibrate, bargs.return_record = False, True
    b = bench_block(bargs, synth.WORKLOADS["block8k"], np, torch, fl, synth)
    keep = ("metric", "value", "unit", "steps", "warmup", "ms_per_step", "loops", "roofline", "gemms_all")
    return {k: b[k] for k in keep if k in b}


def decode_summary(args, np, torch, fl, synth):
    """The batched-decode workload (64 sequences x 8192 cached tokens, R=4,
    one new token per sequence through all loops) timed after the prefill
    measurement, 20 steps after 3 warm-up steps, no CPU baseline: its
    throughput, per-loop times, the sparse and dense decode kernels' average
    launch times and the dense kernel's HBM roofline."""
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    dargs = argparse.Namespace(**vars(args))
    dargs.steps, dargs.warmup, dargs.no_cpu_baseline = 20, 3, True
    d = bench_decode(dargs, synth.WORKLOADS["decode64x8k"], np, torch, fl, synth)
    ks = d["kernels"]
    return {
        "metric": d["metric"], "value": d["value"], "unit": d["unit"], "steps": d["steps"],
        "warmup": d["warmup"], "ms_per_step": d["ms_per_step"], "loops": d["loops"],
        "sparse_decode_avg_launch_us": ks.get("decode", {}).get("avg_launch_us"),
        "dense_decode_avg_launch_us": ks.get("decode_dense", {}).get("avg_launch_us"),
        "kernels": ks, "roofline": d["roofline"],
    }


def lazy_flops(loops, d):
    """Algorithmic flops of steps a5-a8 of each loop r >= 2: QK^T and PV over
    the actual (row, selected causal column) pairs, 4d per pair, twice at a
    loop that rebuilds the pruned-column caches (the previous loop's side
    over the same pairs); the column statistics' recompute is overhead."""
    return {L["r"]: 4.0 * d * L["pairs"] * (2 if L["rebuilt"] else 1) for L in loops if L["r"] > 1}


def bench_prefill(args, w, np, torch, fl, synth, cpu=True, steps=None):
    """R loops of the lazy-update attention step on one layer's synthetic
    inputs (resident in HBM): returns the JSON record.

    value: active-query tokens/s of the sparse loops' attention step,
    sum_{r>=2} n_r over the time of steps a5-a8 (column selection,
    pruned-column caches, sparse attention, column statistics) of loops
    2..R; steps a1-a4 (statistic, selection, quantisation) and loop 1 (the
    dense producer) are reported beside it.  Phases are timed by HIP events
    the library records on the launch stream (no per-kernel events in that
    run); a second run of the same steps records every kernel."""
    steps = steps or args.steps
    t0 = time.time()
    inp = synth.generate(w)
    log(f"[bench] generated {w.name} inputs in {time.time() - t0:.1f}s")
    dt = inp["dtype"]

    def dev(a):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    D = {k: [dev(a) for a in inp[k]] for k in ("h", "q", "k", "v")}
    N, H, d, R = w.N, w.H, w.d, w.R
    n_act = [N]
    for r in range(1, R):
        n_act.append(min(n_act[-1], max(1, int(np.ceil(w.rho[r] * N - 1e-9)))))
    mode = {"auto": fl.FL_DEQ_AUTO, "once": fl.FL_DEQ_ONCE, "in_tile": fl.FL_DEQ_IN_TILE}[args.mode]
    ts, cs = stat_kinds(args, fl)
    run = fl.LoopRunner(N, H, d, w.g, R, w.n_sink, n_act, w.kcols, w.bits,
                        dtype=torch.bfloat16 if dt == "bf16" else torch.float32, mode=mode,
                        token_stat=ts, col_stat=cs, quant=quant_scheme(args, fl))
    stream = torch.cuda.current_stream()

    def loop(r):
        hp = D["h"][r - 2] if r > 1 else None
        qp = D["q"][r - 2] if r > 1 else None
        run.step(r, D["h"][r - 1], hp, D["q"][r - 1], D["k"][r - 1], D["v"][r - 1], qp)

    def step(events=None):
        for r in range(1, R + 1):
            if events is not None:
                events[r - 1].record(stream)
            loop(r)
        if events is not None:
            events[R].record(stream)

    log(f"[bench] inputs resident; n_active={n_act} k={w.kcols}")
    # ---- warmup ----
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    # algorithmic work per loop from the actual index sets
    loops = []
    for r in range(1, R + 1):
        act = run.active[r - 1]
        sel = run.sel_used(r)
        pairs, _ = pairs_per_head(torch, act, sel, N)
        if sel is None:
            pairs *= H
        rebuilt = r > 1 and run.k_used(r) < run.k_used(r - 1)
        colstat = r < R and w.kcols[r] < run.k_used(r)
        loops.append(dict(r=r, n=n_act[r - 1], k=run.k_used(r), pairs=pairs, rebuilt=rebuilt,
                          colstat=colstat))
    log("[bench] warmup done")

    # ---- timed region: loop phases only ----
    fl.fl_timing_report()              # discard warmup records
    fl.fl_timing_enable(2)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(R + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    # the phases of each step read back after it (GPU event times; the host
    # waits between steps); figures are medians over the timed steps
    t_start = time.perf_counter()
    per_step = []
    for s in range(steps):
        step(evs[s])
        torch.cuda.synchronize()
        per_step.append(fl.fl_timing_report())
    wall = time.perf_counter() - t_start
    fl.fl_timing_enable(0)
    loop_ms = np.array([[evs[s][r].elapsed_time(evs[s][r + 1]) for r in range(R)]
                        for s in range(steps)])
    ms_per_step = float(np.median(loop_ms.sum(axis=1)))

    def phase_ms(ph, r, part):
        c, ms = ph.get(f"loop{r}.{part}", (0, 0.0))
        assert c == 1, f"phase loop{r}.{part}: {c} records in one step"
        return ms

    a58_steps = np.array([[phase_ms(ph, r, "a5-a8") for r in range(2, R + 1)] for ph in per_step])
    a14_steps = np.array([[phase_ms(ph, r, "a1-a4") for r in range(2, R + 1)] for ph in per_step])
    a58 = {r: float(np.median(a58_steps[:, r - 2])) for r in range(2, R + 1)}
    a14 = {r: float(np.median(a14_steps[:, r - 2])) for r in range(2, R + 1)}
    lazy_tokens = sum(n_act[1:])
    a58_ms = float(np.median(a58_steps.sum(axis=1))) if R > 1 else 0.0
    a14_ms = float(np.median(a14_steps.sum(axis=1))) if R > 1 else 0.0
    value = lazy_tokens / (a58_ms / 1e3) if R > 1 else None

    # ---- second run of the same steps: every kernel timed ----
    ktab = {}
    if not args.no_kernel_timing:
        fl.fl_timing_enable(1)
        for s in range(steps):
            step()
        torch.cuda.synchronize()
        fl.fl_timing_enable(0)
        ktab = fl.fl_timing_report()

    # per-kernel table: "loop<r>.<phase>/<kernel>" (kernels outside a loop phase
    # have no prefix); aggregated per kernel name over the lazy loops' a5-a8
    kernels = {}
    for name, (cnt, ms) in ktab.items():
        kernels[name] = dict(launches_per_step=cnt / steps, ms_per_step=round(ms / steps, 4),
                             avg_launch_us=round(1e3 * ms / max(cnt, 1), 2))
    lazy_k = {}
    for name, (cnt, ms) in ktab.items():
        if "/" not in name:
            continue
        pfx, kname = name.split("/", 1)
        r = int(pfx[4:pfx.index(".")])
        if r >= 2 and pfx.endswith("a5-a8"):
            e = lazy_k.setdefault(kname, [0, 0.0, []])
            e[0] += cnt; e[1] += ms; e[2].append(r)

    # ---- rooflines ----
    fl_r = lazy_flops(loops, d)
    F_metric = sum(fl_r.values())
    ach_m = F_metric / (a58_ms / 1e3) / 1e12 if a58_ms else None
    roof_metric = dict(work="steps a5-a8 of loops 2..R: 4d flops per (active row, selected causal "
                            "column) pair, twice at a rebuild", bound="mfma", flops_per_step=F_metric,
                       ms_per_step=round(a58_ms, 4), achieved=round(ach_m, 2) if ach_m else None,
                       peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                       frac=round(ach_m / PEAK_BF16_TFLOPS, 4) if ach_m else None)

    def kernel_flops(kname):
        """Algorithmic flops of one lazy-loop kernel per step, over the loops
        it ran in (attn_ad_rb: the cache rebuild and the attention of the
        same pairs, one launch)."""
        per_pair = {"attn_split": 4.0, "attn": 4.0, "attn_ad": 4.0, "attn_rebuild": 4.0,
                    "attn_rebuild_split": 4.0, "attn_ad_rebuild": 4.0, "attn_ad_rb": 8.0,
                    "colstat": 2.0, "colstat_split": 2.0}.get(kname)
        if per_pair is None or kname not in lazy_k:
            return None     # (the additive rebuild's pairs are the pruned ones, not counted here)
        ran = set(lazy_k[kname][2])
        return sum(per_pair * d * L["pairs"] for L in loops if L["r"] in ran)

    roofline = None
    if lazy_k:
        dom = max(lazy_k, key=lambda k: lazy_k[k][1])
        cnt, ms, _ = lazy_k[dom]
        fk = kernel_flops(dom)
        sym = KERNEL_SYMBOL.get(dom, dom)
        if fk:
            # fk: flops per step; cnt launches over `steps` steps taking ms
            ach = fk / (ms / steps / 1e3) / 1e12
            roofline = dict(kernel=dom, kernel_symbol=sym, bound="mfma", achieved=round(ach, 2),
                            peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(ach / PEAK_BF16_TFLOPS, 4),
                            traffic=kernel_traffic(w.name, sym),
                            flops_per_launch=round(fk * steps / cnt, 1), launches_per_step=cnt / steps,
                            avg_launch_us=round(1e3 * ms / cnt, 2))
        else:
            roofline = dict(kernel=dom, kernel_symbol=sym, bound="hbm", achieved=None, peak=PEAK_HBM_GBS,
                            unit="GB/s", frac=None, traffic=None, avg_launch_us=round(1e3 * ms / cnt, 2))
    lazy_kernels = {k: dict(loops=sorted(set(v[2])), launches_per_step=v[0] / steps,
                            ms_per_step=round(v[1] / steps, 4), avg_launch_us=round(1e3 * v[1] / v[0], 2),
                            **({"tflops": round(kernel_flops(k) / (v[1] / steps / 1e3) / 1e12, 2)}
                               if kernel_flops(k) else {}))
                    for k, v in lazy_k.items()}
    # loop 1's dense attention (the step's costliest kernel), for context
    roof_l1 = None
    k1 = ktab.get("loop1.a5-a8/attn")
    if k1:
        f1 = 4.0 * d * loops[0]["pairs"]
        a1 = f1 / (k1[1] / k1[0] / 1e3) / 1e12
        roof_l1 = dict(kernel="attn", kernel_symbol=KERNEL_SYMBOL["attn"], achieved=round(a1, 2),
                       peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(a1 / PEAK_BF16_TFLOPS, 4),
                       avg_launch_us=round(1e3 * k1[1] / k1[0], 2),
                       traffic=kernel_traffic(w.name, KERNEL_SYMBOL["attn"]))

    # ---- KV bytes per token (codes + scales, and with index metadata) ----
    HD = H * d
    kv_codes = 2 * N * (HD + 4 * HD // w.g)
    meta = 0
    for r in range(2, R + 1):
        kv_codes += 2 * n_act[r - 1] * (HD * w.bits[r - 1] // 8 + 4 * HD // w.g)
        meta += 4 * n_act[r - 1] + 4 * N          # row list + slot map
    kv = dict(codes_scales=round(kv_codes / N, 1), with_metadata=round((kv_codes + meta) / N, 1),
              bf16_all_loops=2 * HD * 2 * R, ratio=round(2 * HD * 2 * R / (kv_codes / N), 2))

    out = {
        "metric": METRIC,
        "value": round(value, 1) if value else None,
        "unit": "active-query tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "N": N, "H": H, "d": d, "R": R, "g": w.g,
                   "active_per_loop": n_act, "k_per_loop": [L["k"] for L in loops],
                   "bits_per_loop": w.bits, "n_sink": w.n_sink, "dequant": args.mode,
                   "token_stat": args.token_stat, "col_stat": args.col_stat,
                   "quant": args.quant},
        "value_def": "sum_{r=2..R} n_r / time of steps a5-a8 of loops 2..R (median over the timed steps)",
        "a5_a8_ms": {f"loop{r}": round(v, 4) for r, v in a58.items()},
        "a1_a4": dict(ms={f"loop{r}": round(v, 4) for r, v in a14.items()},
                      tokens_per_s=round(lazy_tokens / (a14_ms / 1e3), 1) if a14_ms else None),
        "lazy_loops_tokens_per_s": round(lazy_tokens / ((a14_ms + a58_ms) / 1e3), 1) if R > 1 else None,
        "step_tokens_per_s": round(sum(n_act) / (ms_per_step / 1e3), 1),
        "loops": [dict(r=L["r"], n=L["n"], k=L["k"], ms=round(float(np.median(loop_ms[:, i])), 4),
                       pairs=L["pairs"], rebuilt=L["rebuilt"], colstat=L["colstat"])
                  for i, L in enumerate(loops)],
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "roofline_metric": roof_metric,
        "roofline_loop1_attn": roof_l1,
        "lazy_kernels": lazy_kernels,
        "kernels": kernels,
        "kv_bytes_per_token": kv,
    }

    log(f"[bench] timed {steps} steps: {ms_per_step:.3f} ms/step; a5-a8 of loops 2..{R}: "
        f"{a58_ms:.3f} ms -> {value / 1e6 if value else 0:.2f} M tokens/s")
    if cpu and R > 1:
        out["cpu_baseline"] = cpu_baseline(w, inp, run, n_act, loops, args.cpu_rows, torch, np,
                                           D, rel=args.token_stat == "rel",
                                           vw=args.col_stat == "vnorm", asym=args.quant == "asym")
    return out


def bench_sweep(args, w, np, torch, fl, synth):
    """Depth and length sweeps of the lazy-update step (paper Fig. 6 and
    Fig. 7): --sweep length runs the workload's recipe at N = 4K..32K with its
    column budgets and kept fractions; --sweep depth runs the deep recipe
    truncated to its first R = 4, 8, 16, 32 loops.  One JSON line with
    tokens/s, step time and KV bytes per token per point."""
    pts = []
    if args.sweep == "length":
        for N in (4096, 8192, 16384, 32768):
            kc = [N] + [min(c, N) for c in w.kcols[1:]]
            pts.append(w.scaled(N=N, kcols=kc, name=f"{w.name}-N{N}"))
    else:
        base = synth.WORKLOADS["depth32x8k"] if w.R < 32 else w
        for R in (4, 8, 16, 32):
            pts.append(base.scaled(R=R, rho=base.rho[:R], kcols=base.kcols[:R], bits=base.bits[:R],
                                   name=f"{base.name}-R{R}"))
    rows = []
    t = time.perf_counter()
    for p in pts:
        o = bench_prefill(args, p, np, torch, fl, synth, cpu=False)
        rows.append(dict(N=p.N, R=p.R, value=o["value"], ms_per_step=o["ms_per_step"],
                         lazy_loops_tokens_per_s=o["lazy_loops_tokens_per_s"],
                         active_tokens=sum(o["config"]["active_per_loop"]),
                         kv_bytes_per_token=o["kv_bytes_per_token"],
                         dominant=(o["roofline"] or {}).get("kernel"),
                         frac=(o["roofline"] or {}).get("frac")))
        log(f"[bench] sweep point N={p.N} R={p.R}: {o['value']:.0f} tok/s, {o['ms_per_step']:.2f} ms")
    out = {"metric": f"{args.sweep} sweep of the lazy-update attention step (active-query tokens/s)",
           "value": rows[-1]["value"], "unit": "active-query tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": rows[-1]["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": pts[-1].name, "sweep": args.sweep, "quant": args.quant},
           "points": rows, "wall_s": round(time.perf_counter() - t, 1)}
    print(json.dumps(out), flush=True)


def quant_scheme(args, fl):
    return fl.FL_QUANT_ASYM if args.quant == "asym" else fl.FL_QUANT_ABSMAX


def oracle_level(oracle, x, prev, g, bits, asym, per_channel):
    """One cache level's reconstruction by the oracle's quantiser."""
    if asym:
        return oracle.quantize_rows_asym(x, prev, g, bits, per_channel)[3]
    return oracle.quantize_rows(x, prev, g, bits)[3]


def stat_kinds(args, fl):
    ts = fl.FL_TOKEN_STAT_REL if args.token_stat == "rel" else fl.FL_TOKEN_STAT_ABS
    cs = fl.FL_COL_STAT_VNORM if args.col_stat == "vnorm" else fl.FL_COL_STAT_MASS
    return ts, cs


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, inp, run, n_act, loops, m, torch, np, D, rel=False, vw=False, asym=False):
    """The oracle, as is, on the metric's work: steps a5-a8 of loops 2..R
    (column selection in full; pruned-column caches, sparse attention and
    column statistics on m evenly spaced active rows per loop, all heads),
    after a warm-up, with steps a1-a4 (statistic, selection, quantisation)
    timed in full beside them.  Loop 1's products are computed once and not
    timed.  The sampled rows use the GPU run's index sets and the loop state
    it left after the previous loop (one extra untimed pass, loop by loop);
    per-row work is independent, so a loop's a6-a8 time scales by n_r / m."""
    import oracle

    t_all = time.time()
    x = {k: [synth_f32(a, inp["dtype"], np) for a in inp[k]] for k in ("h", "q", "k", "v")}
    N, H, d, g, R = w.N, w.H, w.d, w.g, w.R
    sm = np.float32(1.0 / np.sqrt(d))
    acts = [run.active[r].cpu().numpy().copy() for r in range(R)]
    sels = [None if run.sel_used(r + 1) is None else run.sel_used(r + 1).cpu().numpy().copy()
            for r in range(R)]
    samp = {r: acts[r - 1][np.linspace(0, n_act[r - 1] - 1, min(m, n_act[r - 1])).astype(np.int64)]
            for r in range(2, R + 1)}
    # GPU state after each loop at the next loop's sampled rows (untimed)
    snap = {}
    for r in range(1, R + 1):
        hp = D["h"][r - 2] if r > 1 else None
        qp = D["q"][r - 2] if r > 1 else None
        run.step(r, D["h"][r - 1], hp, D["q"][r - 1], D["k"][r - 1], D["v"][r - 1], qp)
        torch.cuda.synchronize()
        if r < R:
            idx = torch.from_numpy(samp[r + 1].astype(np.int64)).cuda()
            snap[r + 1] = dict(lse=run.lse.index_select(0, idx).cpu().numpy(),
                               mu=run.mass_u.index_select(0, idx).cpu().numpy(),
                               ou=run.out_u.index_select(0, idx).cpu().numpy(),
                               cstat=(run.col_stat[r - 1][:, : loops[r - 1]["k"]].cpu().numpy().copy()
                                      if loops[r]["rebuilt"] else None))
    khat = oracle_level(oracle, x["k"][0], None, g, w.bits[0], asym, True)
    vhat = oracle_level(oracle, x["v"][0], None, g, w.bits[0], asym, False)
    # warm-up: every oracle function once on a few rows
    few = samp[2][:4]
    oracle.delta_norm(x["h"][1], x["h"][0], few, relative=rel)
    oracle.attend(x["q"][1], khat, vhat, few, sels[1], sm, snap[2]["mu"][:4], snap[2]["ou"][:4])
    per_loop, t58_tot, t14_tot = [], 0.0, 0.0
    for r in range(2, R + 1):
        A_prev, A, S, S_prev = acts[r - 2], acts[r - 1], sels[r - 1], sels[r - 2]
        sn = snap[r]
        t = time.perf_counter()
        stat = oracle.delta_norm(x["h"][r - 1], x["h"][r - 2], A_prev, relative=rel)
        oracle.top_select(stat, n_act[r - 1], A_prev)
        kr = oracle_level(oracle, x["k"][r - 1][A], khat[A], g, w.bits[r - 1], asym, True)
        vr = oracle_level(oracle, x["v"][r - 1][A], vhat[A], g, w.bits[r - 1], asym, False)
        khat_n = khat.copy(); khat_n[A] = kr
        vhat_n = vhat.copy(); vhat_n[A] = vr
        t14 = time.perf_counter() - t
        t = time.perf_counter()
        if loops[r - 1]["rebuilt"]:
            oracle.select_columns(sn["cstat"], S_prev, loops[r - 1]["k"], w.n_sink)
        t5 = time.perf_counter() - t
        rows = samp[r]
        t = time.perf_counter()
        if loops[r - 1]["rebuilt"]:
            first = S_prev is None
            mu, ou = oracle.unselected_cache(x["q"][r - 2], khat, vhat, rows, S_prev, S, sn["lse"], sm,
                                             None if first else sn["mu"], None if first else sn["ou"])
        else:
            mu, ou = sn["mu"], sn["ou"]
        o, l = oracle.attend(x["q"][r - 1], khat_n, vhat_n, rows, S, sm, mu, ou)
        if loops[r - 1]["colstat"]:
            oracle.column_stats(x["q"][r - 1], khat_n, rows, S, l, sm, mu, vhat=vhat_n if vw else None)
        t68 = time.perf_counter() - t
        t58 = t5 + t68 * len(A) / len(rows)
        per_loop.append(dict(r=r, n=len(A), a1_a4_s=round(t14, 3), a5_s=round(t5, 3),
                             sampled_rows=len(rows), a6_a8_sampled_s=round(t68, 3),
                             a5_a8_s=round(t58, 3)))
        t58_tot += t58
        t14_tot += t14
        khat, vhat = khat_n, vhat_n
        log(f"[bench] cpu oracle loop {r}: a1-a4 {t14:.2f}s, a5 {t5:.2f}s, a6-a8 on {len(rows)} rows "
            f"{t68:.2f}s")
    lazy = sum(n_act[1:])
    return {"value": round(lazy / t58_tot, 1), "unit": "active-query tokens/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": (f"steps a5-a8 of loops 2..{R} of {w.name} (the metric's work): column "
                       f"selection in full; pruned-column caches, attention and column statistics "
                       f"on {m} evenly spaced active rows per loop (all {H} heads), scaled to n_r "
                       f"rows; after a warm-up"),
            "a5_a8_s": round(t58_tot, 3), "a1_a4_tokens_per_s": round(lazy / t14_tot, 1),
            "measured_s": round(time.time() - t_all, 1), "loops": per_loop}


def bench_block(args, w, np, torch, fl, synth):
    """The full looped block: R loops of n_layers layers on each loop's active
    tokens.  value = active tokens pushed through the whole block per second,
    sum_r n_r / step time.  Roofline of the dominant kernel (the costliest
    gathered-row projection; the four take 2*(D*3D + D*D + D*2F + F*D) flops
    per active token and layer), and of the four together."""
    t0 = time.time()
    inp = synth.generate(w)
    log(f"[bench] generated {w.name} weights/inputs in {time.time() - t0:.1f}s")
    N, H, d, R = w.N, w.H, w.d, w.R
    D, F, L = H * d, w.extra["ffn"], w.extra["layers"]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    wdev = [{k: dev(v) for k, v in lw.items()} for lw in inp["layers"]]
    h1 = torch.from_numpy(inp["h1"]).cuda()
    n_act = [N]
    for r in range(1, R):
        n_act.append(min(n_act[-1], max(1, int(np.ceil(w.rho[r] * N - 1e-9)))))
    ts, cs = stat_kinds(args, fl)
    if args.calibrate:
        return bench_calibrate(args, w, h1, wdev, fl, torch, ts, cs)
    run = fl.BlockRunner(N, H, d, w.g, R, w.n_sink, n_act, w.kcols, w.bits, wdev, F,
                         rope_theta=w.extra["theta"], norm_eps=w.extra["eps"], token_stat=ts,
                         col_stat=cs, quant=quant_scheme(args, fl))
    stream = torch.cuda.current_stream()

    def step(events=None):
        run.h.copy_(h1)
        for r in range(1, R + 1):
            if events is not None:
                events[r - 1].record(stream)
            run.step(r)
        if events is not None:
            events[R].record(stream)

    log(f"[bench] block resident: {L} layers, n_active={n_act}, k={w.kcols}")
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    fl.fl_timing_report()
    fl.fl_timing_enable(True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(R + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    fl.fl_timing_enable(False)
    ktab = fl.fl_timing_report()
    loop_ms = np.array([[evs[s_][r].elapsed_time(evs[s_][r + 1]) for r in range(R)]
                        for s_ in range(args.steps)])
    ms_per_step = float(np.mean(loop_ms.sum(axis=1)))
    tokens = sum(n_act)
    per_tok = {"gemm_qkv": 2.0 * D * 3 * D, "gemm_o": 2.0 * D * D, "gemm_gate_up": 2.0 * D * 2 * F,
               "gemm_down": 2.0 * F * D}
    kernels = {}
    # projection timings are named <projection>.w<tile width>; the width
    # varies with the loop's row count, so each projection is also summed
    for name, (cnt, ms) in ktab.items():
        kernels[name] = dict(launches_per_step=cnt / args.steps, ms_per_step=round(ms / args.steps, 4),
                             avg_launch_us=round(1e3 * ms / max(cnt, 1), 2))
    for base in per_tok:
        parts = [(c, m) for nm, (c, m) in ktab.items() if nm.split(".")[0] == base]
        cnt, ms = sum(c for c, _ in parts), sum(m for _, m in parts)
        if cnt and ms > 0:
            kernels[base] = dict(launches_per_step=cnt / args.steps, ms_per_step=round(ms / args.steps, 4),
                                 avg_launch_us=round(1e3 * ms / cnt, 2),
                                 tflops=round(per_tok[base] * tokens * L / (ms / args.steps / 1e3) / 1e12, 2))
    # dominant kernel: the costliest of the projections (a kernel of its own)
    dom = max((k for k in per_tok if k in kernels), key=lambda k: kernels[k]["ms_per_step"], default=None)
    roof = None
    if dom:
        fl_dom = per_tok[dom] * tokens * L
        a_dom = fl_dom / (kernels[dom]["ms_per_step"] / 1e3) / 1e12
        sym = BLOCK_GEMM_SYMBOL.get(dom)
        roof = dict(kernel=dom, kernel_symbol=sym, bound="mfma", achieved=round(a_dom, 2),
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(a_dom / PEAK_BF16_TFLOPS, 4),
                    traffic=kernel_traffic(w.name, sym) if sym else None, flops_per_step=fl_dom,
                    avg_launch_us=kernels[dom]["avg_launch_us"])
    gemm_ms = sum(kernels[k]["ms_per_step"] for k in per_tok if k in kernels)
    gemm_flops = sum(per_tok.values()) * tokens * L
    ach = gemm_flops / (gemm_ms / 1e3) / 1e12 if gemm_ms else None
    out = {
        "metric": "active tokens/s through the token-sparse looped block (24 layers, R=4, 8K)",
        "value": round(tokens / (ms_per_step / 1e3), 1), "unit": "active tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random-init shared weights)",
        "config": {"workload": w.name, "N": N, "layers": L, "hidden": D, "heads": H, "head_dim": d,
                   "ffn": F, "R": R, "active_per_loop": n_act, "k_per_loop": w.kcols,
                   "bits_per_loop": w.bits, "token_stat": args.token_stat,
                   "col_stat": args.col_stat, "quant": args.quant},
        "loops": [dict(r=r + 1, n=n_act[r], ms=round(float(np.mean(loop_ms[:, r])), 3))
                  for r in range(R)],
        "kernels": kernels,
        "roofline": roof,
        "gemms_all": dict(achieved=round(ach, 2) if ach else None, unit="TFLOP/s",
                          frac=round(ach / PEAK_BF16_TFLOPS, 4) if ach else None,
                          flops_per_step=gemm_flops),
        "gemm_flops_dense_equivalent": sum(per_tok.values()) * N * R * L,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_block(w, inp, n_act, np, rel=args.token_stat == "rel",
                                                 vw=args.col_stat == "vnorm",
                                                 asym=args.quant == "asym")
    if getattr(args, "return_record", False):
        return out
    print(json.dumps(out), flush=True)


def cpu_baseline_block(w, inp, n_act, np, m=32, rel=False, vw=False, asym=False):
    """The block oracle's step functions, as they are, on a bounded sample of
    the same workload: the first layer through all R loops.  Token
    selection, RMSNorm, the four projections, RoPE, quantisation and column
    selection run in full; attention, cache rebuild and column statistics run
    on m evenly spaced active rows per loop (all heads) and are extrapolated
    to n_r rows; the layer is extrapolated to the workload's layer count."""
    import oracle
    from oracle import block as ob
    from sparse_attention_kv_amd import synth
    F32 = np.float32
    N, H, d, g, R = w.N, w.H, w.d, w.g, w.R
    D, L = H * d, w.extra["layers"]
    sm = F32(1.0 / np.sqrt(d))
    lw = {k: synth.bf16_bits_to_f32(v) for k, v in inp["layers"][0].items()}
    h = np.array(inp["h1"], F32, copy=True)
    h_entry = h.copy()
    A = np.arange(N, dtype=np.int32)
    khat = vhat = S = cstat = lse = None
    qd = np.zeros((N, H, d), F32)
    total = 0.0
    for r in range(1, R + 1):
        t_full = t_rows = 0.0
        t = time.perf_counter()
        if r > 1:
            stat = oracle.delta_norm(h, h_entry, A, relative=rel)
            A = oracle.top_select(stat, n_act[r - 1], A)
        h_entry = h.copy()
        a = ob.bf16(ob.rmsnorm(h[A], lw["norm1"], w.extra["eps"]))
        qkv = ob.bf16(a @ lw["w_qkv"].T)
        q = ob.bf16(ob.rope(qkv[:, :D].reshape(-1, H, d), A, w.extra["theta"]))
        k = ob.bf16(ob.rope(qkv[:, D:2 * D].reshape(-1, H, d), A, w.extra["theta"]))
        v = np.ascontiguousarray(qkv[:, 2 * D:].reshape(-1, H, d))
        kx = oracle_level(oracle, k, None if r == 1 else khat[A], g, w.bits[r - 1], asym, True)
        vx = oracle_level(oracle, v, None if r == 1 else vhat[A], g, w.bits[r - 1], asym, False)
        kh = kx if r == 1 else khat.copy()
        vh = vx if r == 1 else vhat.copy()
        if r > 1:
            kh[A] = kx; vh[A] = vx
        qn = qd.copy(); qn[A] = q
        S_new = S
        if r > 1 and w.kcols[r - 1] < (N if S is None else S.shape[1]):
            S_new = oracle.select_columns(cstat, S, w.kcols[r - 1], w.n_sink)
        t_full += time.perf_counter() - t
        samp = A[np.linspace(0, len(A) - 1, min(m, len(A))).astype(np.int64)]
        t = time.perf_counter()
        if r > 1 and S_new is not S:
            oracle.unselected_cache(qd, khat, vhat, samp, S, S_new, lse[samp], sm)
        o, l_s = oracle.attend(qn, kh, vh, samp, S_new, sm)
        if r < R:
            cstat_s = oracle.column_stats(qn, kh, samp, S_new, l_s, sm, vhat=vh if vw else None)
        t_rows = time.perf_counter() - t
        t = time.perf_counter()
        # the rest of the layer on the active rows (outputs of the rows not
        # sampled are zeros here: the projections' cost does not depend on them)
        att = np.zeros((len(A), D), F32)
        h[A] += (ob.bf16(att) @ lw["w_o"].T).astype(F32)
        b = ob.bf16(ob.rmsnorm(h[A], lw["norm2"], w.extra["eps"]))
        gu = (b @ lw["w_gu"].T).astype(F32)
        h[A] += (ob.bf16(ob.silu(gu[:, 0::2]) * gu[:, 1::2]) @ lw["w_down"].T).astype(F32)
        t_full += time.perf_counter() - t
        total += t_full + t_rows * len(A) / len(samp)
        log(f"[bench] cpu oracle block loop {r}: full {t_full:.2f}s, {len(samp)} rows {t_rows:.2f}s")
        # state for the next loop (column statistic from the sampled rows,
        # full-size so the selection runs at its real size)
        khat, vhat, qd, S = kh, vh, qn, S_new
        lse = np.zeros((N, H), F32)
        if r < R:
            cstat = np.zeros((H, N if S is None else S.shape[1]), F32)
            cstat[:, :cstat_s.shape[1]] = cstat_s
    step_s = total * L
    return {"value": round(sum(n_act) / step_s, 2), "unit": "active tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": (f"layer 1 of {L} through all {R} loops: selection, norms, projections, RoPE, "
                       f"quantisation and column selection in full; attention, cache rebuild and column "
                       f"statistics on {m} evenly spaced active rows per loop (all {H} heads), "
                       f"extrapolated to n_r rows, then x{L} layers"),
            "extrapolated_step_s": round(step_s, 1)}


def bench_calibrate(args, w, h1, wdev, fl, torch, ts, cs):
    """Retention calibration (App. E reading: smallest ratio per loop with
    hidden-state error below 5% against the all-tokens run) of the block
    workload, timed end to end: value = candidate loops evaluated per second."""
    from sparse_attention_kv_amd import calibrate
    N, R = w.N, w.R
    run = fl.BlockRunner(N, w.H, w.d, w.g, R, w.n_sink, [N] * R, w.kcols, w.bits, wdev,
                         w.extra["ffn"], rope_theta=w.extra["theta"], norm_eps=w.extra["eps"],
                         token_stat=ts, col_stat=cs, row_capacity=[N] * R)
    grid = [0.1 * i for i in range(1, 11)]
    calibrate.calibrate_retention(run, h1, [1.0], tol=0.05)      # warm-up (one ratio)
    torch.cuda.synchronize()
    t = time.perf_counter()
    res = calibrate.calibrate_retention(run, h1, grid, tol=0.05)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t
    loops_run = R + sum(r * len(tr) for r, tr in res["trials"].items())
    out = {"metric": "retention calibration of the looped block (loops evaluated per second)",
           "value": round(loops_run / wall, 2), "unit": "block loops/s", "n_gpus": 1,
           "steps": 1, "warmup": 1, "ms_per_step": round(wall * 1e3, 1), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (random-init shared weights)",
           "config": {"workload": w.name, "N": N, "layers": w.extra["layers"], "R": R,
                      "grid": [round(g_, 2) for g_ in grid], "bound": 0.05,
                      "token_stat": args.token_stat, "col_stat": args.col_stat},
           "calibrated": {"rho": [round(x, 2) for x in res["rho"]], "n_active": res["n_active"],
                          "err": [round(e, 5) for e in res["err"]]},
           "trials": {str(r): [[round(c, 2), n, round(e, 5)] for c, n, e in tr]
                      for r, tr in res["trials"].items()}}
    print(json.dumps(out), flush=True)


def bench_quant_study(args, w, np, torch, fl, synth):
    """Residual vs direct quantisation error by loop (Sec. 3.3, Fig. 2(c),
    Table 2's per-loop direct quantisation) on the workload's K/V with every
    token active: the paper's quantiser (INT4 asymmetric, keys per channel,
    values per token) and the absmax int8 base + int4/int2 residual one."""
    from sparse_attention_kv_amd import quant_study
    if w.kind != "prefill":
        raise SystemExit("--quant-study needs a prefill workload")
    inp = synth.generate(w)

    def dev(a):
        if inp["dtype"] == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    ks = [dev(a) for a in inp["k"]]
    vs = [dev(a) for a in inp["v"]]
    base = synth.WORKLOADS[w.name].bits
    res = {}
    t = time.perf_counter()
    for name, scheme, bits in (("asym_int4", fl.FL_QUANT_ASYM, [4] * w.R),
                               ("absmax_spec", fl.FL_QUANT_ABSMAX, base)):
        rows = quant_study.residual_vs_direct(ks, vs, w.g, bits, scheme)
        res[name] = dict(bits=bits, loops=[{k: (round(v, 6) if isinstance(v, float) else v)
                                            for k, v in r.items()} for r in rows])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t
    ratios = [r[kv + "_dir"] / r[kv + "_res"] for r in res["asym_int4"]["loops"][1:]
              for kv in ("k", "v") if r[kv + "_res"] > 0]
    out = {"metric": "direct / residual relative reconstruction error of the per-loop KV "
                     "(paper's INT4 quantiser, loops >= 2, geometric mean over K and V)",
           "value": round(float(np.exp(np.mean(np.log(ratios)))), 3) if ratios else None,
           "unit": "x", "n_gpus": 1, "steps": 1,
           "warmup": 0, "ms_per_step": round(wall * 1e3, 1), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": inp["dtype"], "data": "synthetic",
           "config": {"workload": w.name, "N": w.N, "H": w.H, "d": w.d, "R": w.R, "g": w.g,
                      "tokens_active": "all"},
           "schemes": res}
    print(json.dumps(out), flush=True)


def bench_decode(args, w, np, torch, fl, synth):
    """Batched decode: B sequences with resident loop-indexed prefix caches;
    a step decodes one new token per sequence through all R loops (loop 1
    dense over the prefix, later loops on the selected columns, the cached
    mass / partial output rebuilt when the column set shrinks).
    value = decoded tokens per second, B / step time.  The dominant kernel
    (the dense first loop) is bounded by HBM: its algorithmic bytes are the
    prefix's int8 K/V codes and fp32 group scales, the column statistic it
    writes, and the token's q/k/v in and output out."""
    from concurrent.futures import ThreadPoolExecutor
    B, N, H, d, R, g = w.extra["B"], w.N, w.H, w.d, w.R, w.g
    asym = args.quant == "asym"
    n_act = [N]
    for r in range(1, R):
        n_act.append(min(n_act[-1], max(1, int(np.ceil(w.rho[r] * N - 1e-9)))))
    run = fl.DecodeRunner(B, N, H, d, g, R, w.n_sink, n_act, w.kcols, w.bits, quant=quant_scheme(args, fl))

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    t0 = time.time()
    tok = {key: np.empty((R, B, H, d), np.uint16) for key in ("q_new", "k_new", "v_new")}
    nthr = min(16, os.cpu_count() or 1)
    sample_inputs = {}
    n_cpu = 0 if args.no_cpu_baseline else 2
    with ThreadPoolExecutor(nthr) as ex:
        for b0 in range(0, B, nthr):
            futs = [ex.submit(synth.gen_decode_seq, w, b) for b in range(b0, min(B, b0 + nthr))]
            for i, f in enumerate(futs):
                b, x = b0 + i, f.result()
                st = [None] + [torch.from_numpy(a).cuda() for a in x["stat"][1:]]
                run.load_sequence(b, [dev(a) for a in x["k"]], [dev(a) for a in x["v"]], st)
                for key in tok:
                    for r in range(R):
                        tok[key][r, b] = x[key][r]
                if b < n_cpu:
                    sample_inputs[b] = x
            torch.cuda.synchronize()
    log(f"[bench] {B} sequences x {N} tokens drawn and cached in {time.time() - t0:.1f}s")
    T = {key: [dev(tok[key][r]) for r in range(R)] for key in tok}
    stream = torch.cuda.current_stream()

    def step(events=None):
        for r in range(1, R + 1):
            if events is not None:
                events[r - 1].record(stream)
            prev = [T[key][r - 2] if r > 1 else None for key in ("q_new", "k_new", "v_new")]
            run.step(r, T["q_new"][r - 1], T["k_new"][r - 1], T["v_new"][r - 1], *prev)
        if events is not None:
            events[R].record(stream)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    fl.fl_timing_report()
    fl.fl_timing_enable(True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(R + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    fl.fl_timing_enable(False)
    ktab = fl.fl_timing_report()
    loop_ms = np.array([[evs[s_][r].elapsed_time(evs[s_][r + 1]) for r in range(R)]
                        for s_ in range(args.steps)])
    ms_per_step = float(np.median(loop_ms.sum(axis=1)))

    # algorithmic bytes per launch
    G = d // g
    if asym:
        # K+V codes, the values' scale and offset per g channels, and the keys'
        # per-channel scale and offset shared by g rows (their share per row)
        col_b = [2 * d * b_ // 8 + 2 * G * 4 + 2 * d * 4 // g for b_ in w.bits]
    else:
        col_b = [2 * d * b_ // 8 + 2 * G * 4 for b_ in w.bits]   # K+V codes + scales of one row
    tok_io = 3 * d * 2 + d * 4 + 4                               # q,k,v in; out, lse out
    need_c1 = R > 1 and w.kcols[1] < N
    dense_bytes = B * H * (N * col_b[0] + (N * 4 if need_c1 else 0) + tok_io)
    # sparse loops: selected columns' present levels (from the GPU's sets)
    sparse_bytes = {}
    for r in range(2 if not asym else R + 1, R + 1):   # (asym: scattered key groups, not counted)
        sel = run.sel_used(r)
        if sel is None:
            continue
        kk = sel.shape[-1]
        j = sel.to(torch.int64).reshape(B, -1)
        present = torch.ones_like(j, dtype=torch.bool)
        tot = col_b[0] * j.numel()
        for l in range(1, r):
            present &= torch.gather(run.slot[l].to(torch.int64), 1, j) >= 0
            tot += (col_b[l] + 4) * int(present.sum().item())   # + the slot lookup
        io = B * H * (kk * 4 + tok_io + d * 4 + 4)               # sel, token io, O_U / M_U in
        sparse_bytes[r] = tot + io
    kernels = {}
    for name, (cnt, ms) in ktab.items():
        kernels[name] = dict(launches_per_step=cnt / args.steps, ms_per_step=round(ms / args.steps, 4),
                             avg_launch_us=round(1e3 * ms / max(cnt, 1), 2))
    roof = None
    if "decode_dense" in kernels:
        kd = kernels["decode_dense"]
        per_launch = dense_bytes
        ach = per_launch / (kd["avg_launch_us"] / 1e6) / 1e9
        kd["gbs"] = round(ach, 1)
        # the asymmetric kernel is specialised on the base level's code width
        sym = (f"k_decode<128, 0, false, true, true, {w.bits[0]}>" if asym
               else KERNEL_SYMBOL["decode_dense"])
        roof = dict(kernel="decode_dense", kernel_symbol=sym, bound="hbm", achieved=round(ach, 1),
                    peak=PEAK_HBM_GBS, unit="GB/s", frac=round(ach / PEAK_HBM_GBS, 4),
                    traffic=kernel_traffic(w.name, sym), bytes_per_launch=per_launch)
    if "decode" in kernels and sparse_bytes:
        kd = kernels["decode"]
        avg_b = sum(sparse_bytes.values()) / len(sparse_bytes)
        kd["gbs"] = round(avg_b / (kd["avg_launch_us"] / 1e6) / 1e9, 1)
        kd["bytes_per_launch_avg"] = int(avg_b)
    cpu = None
    if n_cpu:
        from oracle import decode as od
        import oracle
        f = synth.bf16_bits_to_f32
        sched = w.sched()
        if asym:
            sched["quant"] = "asym"
        t_or = 0.0
        for b, x in sample_inputs.items():
            cache = od.build_cache([f(a) for a in x["k"]], [f(a) for a in x["v"]], x["stat"], sched)
            t1 = time.time()
            od.run_decode(cache, [f(a) for a in x["q_new"]], [f(a) for a in x["k_new"]],
                          [f(a) for a in x["v_new"]], sched)
            t_or += time.time() - t1
        cpu = dict(value=round(len(sample_inputs) / t_or, 3), unit="decoded tokens/s",
                   cores=oracle.num_threads(), kind="oracle",
                   sample=f"{len(sample_inputs)} of the {B} sequences, all R={R} loops of the new "
                          f"token (cache already built, as on the GPU)")
    out = {
        "metric": f"decoded tokens/s, {B} sequences x {N} cached tokens, R={R}",
        "value": round(B / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "unsigned min/max codes, f32" if asym else "int8/int4 codes, f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "N": N, "H": H, "d": d, "R": R, "g": g,
                   "active_per_loop": n_act, "k_per_loop": w.kcols, "bits_per_loop": w.bits,
                   "quant": args.quant},
        "loops": [dict(r=r + 1, ms=round(float(np.median(loop_ms[:, r])), 4)) for r in range(R)],
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    return out


def bench_generate(args, w, np, torch, fl, synth):
    """Generation-time decode with the paper's timing protocol (Sec. 5
    speedup measurement: 16 generated tokens of warm-up, then the average
    per-token latency over the next 16).  B sequences with resident prompt
    caches; each generated token runs R loops over the cache plus a bf16
    window of the most recent 64 generated tokens (App. E); once the window
    is full, the token leaving it is appended to the quantised cache first
    (under --quant asym the oldest g tokens leave together, as one key group).
    value = generated tokens/s over the timed tokens, B * timed / time."""
    from concurrent.futures import ThreadPoolExecutor
    B, N, H, d, R, g = w.extra["B"], w.N, w.H, w.d, w.R, w.g
    n_warm, n_timed = args.gen_warmup, args.gen_timed
    n_gen = n_warm + n_timed
    n_act = [N]
    for r in range(1, R):
        n_act.append(min(n_act[-1], max(1, int(np.ceil(w.rho[r] * N - 1e-9)))))
    run = fl.DecodeRunner(B, N, H, d, g, R, w.n_sink, n_act, w.kcols, w.bits, gen_tokens=n_gen,
                          window=64, quant=quant_scheme(args, fl))

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    t0 = time.time()
    tok = {key: np.empty((n_gen, R, B, H, d), np.uint16) for key in ("gen_q", "gen_k", "gen_v")}
    nthr = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthr) as ex:
        for b0 in range(0, B, nthr):
            futs = [ex.submit(synth.gen_decode_seq, w, b, n_gen) for b in range(b0, min(B, b0 + nthr))]
            for i, f in enumerate(futs):
                b, x = b0 + i, f.result()
                st = [None] + [torch.from_numpy(a).cuda() for a in x["stat"][1:]]
                run.load_sequence(b, [dev(a) for a in x["k"]], [dev(a) for a in x["v"]], st)
                for key in tok:
                    for t in range(n_gen):
                        for r in range(R):
                            tok[key][t, r, b] = x[key][t][r]
            torch.cuda.synchronize()
    log(f"[bench] {B} prompts x {N} tokens drawn and cached in {time.time() - t0:.1f}s")
    T = {key: [[dev(tok[key][t, r]) for r in range(R)] for t in range(n_gen)] for key in tok}
    stream = torch.cuda.current_stream()
    for t in range(n_warm):
        run.generate(T["gen_q"][t], T["gen_k"][t], T["gen_v"][t])
    torch.cuda.synchronize()
    fl.fl_timing_report()
    fl.fl_timing_enable(True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_timed + 1)]
    n_before = run.cfg.N
    evs[0].record(stream)
    for i, t in enumerate(range(n_warm, n_gen)):
        run.generate(T["gen_q"][t], T["gen_k"][t], T["gen_v"][t])
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    fl.fl_timing_enable(False)
    ktab = fl.fl_timing_report()
    tok_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(n_timed)]
    ms_per_tok = float(np.mean(tok_ms))
    kernels = {name: dict(launches_per_token=cnt / n_timed, ms_per_token=round(ms / n_timed, 4),
                          avg_launch_us=round(1e3 * ms / max(cnt, 1), 2))
               for name, (cnt, ms) in ktab.items()}
    out = {
        "metric": f"generated tokens/s, {B} sequences x {N}-token prompts, R={R} "
                  f"({n_warm} warm-up tokens, mean over the next {n_timed})",
        "value": round(B / (ms_per_tok / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": n_timed, "warmup": n_warm, "ms_per_step": round(ms_per_tok, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("uint4 codes" if args.quant == "asym" else "int8/int4 codes") + ", bf16 window, f32",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": "generate", "quant": args.quant, "B": B, "N_prompt": N,
                   "H": H, "d": d,
                   "R": R, "g": g, "window": 64, "k_per_loop": w.kcols, "bits_per_loop": w.bits,
                   "context_at_timing": [n_before, run.cfg.N], "window_tokens_at_end": run.win.count - 1},
        "ms_per_token_min_max": [round(min(tok_ms), 4), round(max(tok_ms), 4)],
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def synth_f32(a, dtype, np):
    from sparse_attention_kv_amd import synth
    return synth.to_f32(a, dtype)


if __name__ == "__main__":
    main()
