#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

A step is one moe_layer_forward over the whole routing batch (route, dispatch, grouped SwiGLU
experts, shared experts, combine, statistics) with every input already resident in HBM. The
default workload is the Mixtral-8x7B-shaped layer (T=4096, d=4096, E=8, k=2, M=14336, bf16).

Prints one JSON line: tokens/s, the dominant kernel's roofline (per-launch duration from HIP
events recorded between the library's stages on its stream), per-stage figures, and the CPU
oracle timed on a bounded sample of the same workload.

Timing: W untimed warm-up steps, then K steps between two synchronisations with nothing else
enqueued (``value`` and ``ms_per_step``); then K more steps, each bracketed by two events on the
stream, for the median and spread of the step time; then K more with the library's stage events
for the per-stage times and the roofline kernel's per-launch duration (median over the K steps).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --trace-summary kernel_trace.csv [--skip N]   # per-kernel statistics of a
        rocprofv3 kernel trace, leaving out each kernel's first N launches (the warm-up)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer fwd tokens/sec + % bf16 MFMA peak, Mixtral-8x7B-shaped layer"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_up_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the layer backward")
    ap.add_argument("--backward-steps", type=int, default=3)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="also run one plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time the vendor GEMM (torch.mm -> hipBLASLt) on one dense matrix of "
                         "each expert product's shape, as a reference point (bf16 only)")
    ap.add_argument("--power-probe", action="store_true",
                    help="time moe_expert_ffn on the workload's expert shapes (E groups of kT/E "
                         "rows) with random operands, then with constant ones, and exit")
    ap.add_argument("--trace-summary", default=None,
                    help="print per-kernel statistics of this rocprofv3 kernel_trace.csv and exit")
    ap.add_argument("--skip", type=int, default=0,
                    help="with --trace-summary: leave out each kernel's first N launches")
    return ap.parse_args()


def trace_summary(path: str, skip: int) -> None:
    """Per-kernel launch statistics (µs) of a rocprofv3 kernel trace, each kernel's first `skip`
    launches (the warm-up) left out; a markdown table on stdout."""
    import csv
    import statistics
    durs = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            name = row["Kernel_Name"]
            durs.setdefault(name, []).append(
                (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    rows = []
    for name, v in durs.items():
        kept = v[skip:] if len(v) > skip else v
        rows.append((sum(kept), name, len(v), len(kept), statistics.mean(kept),
                     statistics.median(kept), min(kept), max(kept)))
    rows.sort(reverse=True)
    total = sum(r[0] for r in rows)
    print(f"| kernel | launches (kept) | total µs | % | mean µs | median µs | min µs | max µs |")
    print("|---|---|---|---|---|---|---|---|")
    for tot, name, n, nk, mean, med, lo, hi in rows:
        short = name if len(name) < 140 else name[:137] + "..."
        print(f"| `{short}` | {n} ({nk}) | {tot:.1f} | {100 * tot / total:.2f} | {mean:.2f} | "
              f"{med:.2f} | {lo:.2f} | {hi:.2f} |")


def power_probe(cfg, reps: int = 6) -> None:
    """The grouped expert products (moe_expert_ffn: gate/up + SwiGLU, then down) on E balanced
    groups of kT/E rows at the workload's d and M, with random operands, then all-constant ones
    (same instructions and addresses, far less switching). Prints one JSON line per operand kind
    with the median time of the whole call (both products)."""
    import torch

    import mixture_experts_layer_loss_amd as moe
    dev = torch.device("cuda:0")
    E, d, M = cfg.E, cfg.d, cfg.M
    rows = cfg.k * cfg.T // cfg.E
    offs = torch.arange(0, E + 1, dtype=torch.int32, device=dev) * rows
    g = torch.Generator(device=dev).manual_seed(7)
    for kind in ("random", "constant", "random"):
        if kind == "random":
            X = torch.randn(E * rows, d, device=dev, generator=g).to(torch.bfloat16)
            Wg = (torch.randn(E, M, d, device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
            Wu = (torch.randn(E, M, d, device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
            Wd = (torch.randn(E, d, M, device=dev, generator=g) / M ** 0.5).to(torch.bfloat16)
        else:
            X = torch.full((E * rows, d), 0.5, device=dev, dtype=torch.bfloat16)
            Wg = torch.full((E, M, d), 0.01, device=dev, dtype=torch.bfloat16)
            Wu = Wg.clone()
            Wd = torch.full((E, d, M), 0.01, device=dev, dtype=torch.bfloat16)
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            moe.moe_expert_ffn(X, offs, Wg, Wu, Wd)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        ms.sort()
        med = ms[len(ms) // 2]
        flops = 6.0 * d * M * E * rows
        print(json.dumps({"probe": "expert_ffn", "operands": kind, "groups": E, "rows": rows,
                          "d": d, "M": M, "ms_median": round(med, 4),
                          "tflops": round(flops / (med * 1e-3) / 1e12, 1)}), flush=True)
        del X, Wg, Wu, Wd


def gemm_source_sha() -> str:
    """Hash of the grouped-GEMM kernel source the traffic counters were taken on."""
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "mixture_experts_layer_loss_amd", "csrc", "gemm_bf16.hip"),
              "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """Counter-measured HBM bytes per launch of the gate/up GEMM, if taken on the current source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    if not entry or entry.get("source_sha") != gemm_source_sha():
        return None
    return entry.get("bytes_per_launch")


def blas_reference(cfg, rows: int, dev):
    """The vendor library on the dense equivalents of the two routed expert products: all kept
    rows against ONE weight matrix (no row gather, no per-expert groups, no SwiGLU epilogue), in
    the same operand layout (both operands contiguous along the reduction). A reference point for
    the grouped kernels, not part of a step."""
    import torch
    d, M = cfg.d, cfg.M
    g = torch.Generator(device=dev).manual_seed(5)
    a_up = torch.randn(rows, d, device=dev, dtype=torch.bfloat16, generator=g)
    w_up = torch.randn(2 * M, d, device=dev, dtype=torch.bfloat16, generator=g)
    a_dn = torch.randn(rows, M, device=dev, dtype=torch.bfloat16, generator=g)
    w_dn = torch.randn(d, M, device=dev, dtype=torch.bfloat16, generator=g)

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    up_ms = timed(lambda: torch.mm(a_up, w_up.t()))
    dn_ms = timed(lambda: torch.mm(a_dn, w_dn.t()))
    fl_up, fl_dn = 4.0 * d * M * rows, 2.0 * d * M * rows
    return {"what": "torch.mm (hipBLASLt), dense [rows, K] x [K, N] with the routed products' "
                    "rows, K and N", "rows": rows,
            "gemm_up_ms": round(up_ms, 4), "gemm_up_tflops": round(fl_up / up_ms / 1e9, 1),
            "gemm_down_ms": round(dn_ms, 4), "gemm_down_tflops": round(fl_dn / dn_ms / 1e9, 1)}


def cpu_baseline(cfg, inp, seconds: float):
    """The oracle as it stands, on the first T' tokens of the same inputs (fp64, host BLAS)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O

    shared = [tuple(t for t in s) for s in inp.shared]

    def run(n):
        t0 = time.perf_counter()
        if cfg.routing == "expert":
            O.layer_forward_expert_choice(inp.x[:n], inp.W_r, inp.W_gate, inp.W_up, inp.W_down,
                                          cfg.k, shared=shared, c=cfg.c, renorm=cfg.renorm,
                                          lam=cfg.lam, scoring=cfg.scoring)
        else:
            O.layer_forward(inp.x[:n], inp.W_r, inp.W_gate, inp.W_up, inp.W_down, cfg.k,
                            b=inp.b, shared=shared, c=cfg.c, renorm=cfg.renorm, lam=cfg.lam,
                            scoring=cfg.scoring, gamma=cfg.gamma)
        return time.perf_counter() - t0

    # fixed cost (weight upcasts) plus a per-token cost, from two probes
    p1, p2 = min(cfg.T, 32), min(cfg.T, 96)
    t1, t2 = run(p1), run(p2)
    per_tok = max((t2 - t1) / max(p2 - p1, 1), 1e-6)
    fixed = max(t1 - per_tok * p1, 0.0)
    n = int(min(cfg.T, max(p2, (seconds - fixed) / per_tok)))
    n = max(32, (n // 32) * 32)
    dt = run(n)
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] or [1])
    blas = ", ".join(sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip()
                             for p in pools if p.get("user_api") == "blas"})) or "unknown"
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    note = "" if cfg.c is None else "; capacity applied within the sample"
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens of the same layer (all {cfg.E} experts' weights), "
                      f"fp64 NumPy oracle, {dt:.1f} s{note}",
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model, "blas": blas}


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.skip)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the layer on a single MI355X and "
              "has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_loss_amd as moe
    import workloads

    name = args.workload or workloads.HEADLINE
    cfg = workloads.CONFIGS[name]
    if args.power_probe:
        power_probe(cfg)
        return
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    host = workloads.make_inputs(cfg)
    x = host.x.to(dev)
    W_r = host.W_r.to(dev)
    Wg = host.W_gate.to(dev)
    Wu = host.W_up.to(dev)
    Wd = host.W_down.to(dev)
    b = None if host.b is None else host.b.to(dev)
    sh = host.shared_fused()
    sh = None if sh is None else tuple(t.to(dev) for t in sh)

    layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.M, cfg.S, cfg.c, cfg.renorm, dt, dev,
                         cfg.scoring, cfg.routing)
    out = layer.alloc_outputs(with_bias=b is not None)

    def step():
        layer.forward(x, W_r, Wg, Wu, Wd, b, sh, cfg.lam, cfg.gamma, out=out)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # the step-time distribution: every step between two events on the stream
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for a, b_ in step_ev:
        a.record(stream)
        step()
        b_.record(stream)
    torch.cuda.synchronize()
    step_ms_each = np.array([a.elapsed_time(b_) for a, b_ in step_ev])

    # stage events for every step of a third pass (recorded by the library on its stream)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.STAGE_COUNT)]
              for _ in range(args.steps)]
    for evs in events:
        for ev in evs:
            ev.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        moe.moe_set_stage_events(events[i])
        step()
    torch.cuda.synchronize()
    moe.moe_set_stage_events(None)

    # the balance-loss backward through the router (a separate entry point; not part of a step)
    lb_ws = moe.workspace(moe.make_shape(cfg.T, cfg.d, cfg.E, cfg.k, 8, c=cfg.c, dtype=dt,
                                         scoring=cfg.scoring, routing=cfg.routing),
                          moe.CALL_LOSS_BACKWARD, dev)
    n_fwd = out["counts"]
    for _ in range(2):
        lb = moe.moe_balance_loss_backward(x, W_r, n_fwd, cfg.k, cfg.lam, 1.0, c=cfg.c,
                                           scoring=cfg.scoring, routing=cfg.routing, ws=lb_ws)
    lb_s, lb_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lb_s.record()
    for _ in range(5):
        lb = moe.moe_balance_loss_backward(x, W_r, n_fwd, cfg.k, cfg.lam, 1.0, c=cfg.c,
                                           scoring=cfg.scoring, routing=cfg.routing, ws=lb_ws)
    lb_e.record()
    torch.cuda.synchronize()
    lb_ms = lb_s.elapsed_time(lb_e) / 5
    del lb, lb_ws

    # the full layer backward (token choice): gradients of <dy, y> + aux + z for x, W_r and every
    # expert weight, forward recompute included (a separate entry point; not part of a step)
    bw_ms = None
    train_saved = None
    if not args.no_backward:
        print("[bench] layer backward", file=sys.stderr, flush=True)
        dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator().manual_seed(11)).to(dt).to(dev)
        bw_ws = moe.workspace(moe.make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.M, cfg.S, cfg.c,
                                             cfg.renorm, dt, cfg.scoring, cfg.routing),
                              moe.CALL_LAYER_BACKWARD, dev)
        shared_w = sh
        def bw():
            return moe.moe_layer_backward(x, W_r, Wg, Wu, Wd, dy, cfg.k, b=b, shared=shared_w,
                                          c=cfg.c, renorm=cfg.renorm, lam=cfg.lam, z_coef=1.0,
                                          scoring=cfg.scoring, routing=cfg.routing, ws=bw_ws)
        g = bw()
        torch.cuda.synchronize()
        del g
        bw_s, bw_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bw_s.record()
        for _ in range(args.backward_steps):
            g = bw()
            del g
        bw_e.record()
        torch.cuda.synchronize()
        bw_ms = bw_s.elapsed_time(bw_e) / args.backward_steps
        if cfg.dtype == "bf16":
            # training pair with the forward keeping its fp32 gate/up pre-activations, so that the
            # backward skips recomputing them (the gradients are bit-identical)
            saved = layer.saved_buffer()
            out_s = layer.alloc_outputs(with_bias=b is not None)

            def fwd_save():
                layer.forward(x, W_r, Wg, Wu, Wd, b, sh, cfg.lam, cfg.gamma, out=out_s, saved=saved)

            def bw_saved():
                return moe.moe_layer_backward(x, W_r, Wg, Wu, Wd, dy, cfg.k, b=b, shared=shared_w,
                                              c=cfg.c, renorm=cfg.renorm, lam=cfg.lam, z_coef=1.0,
                                              scoring=cfg.scoring, routing=cfg.routing, ws=bw_ws,
                                              saved=saved)
            fwd_save()
            g = bw_saved()
            torch.cuda.synchronize()
            del g
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
            for _ in range(args.backward_steps):
                fwd_save()
            ev[1].record()
            for _ in range(args.backward_steps):
                g = bw_saved()
                del g
            ev[2].record()
            torch.cuda.synchronize()
            train_saved = (ev[0].elapsed_time(ev[1]) / args.backward_steps,
                           ev[1].elapsed_time(ev[2]) / args.backward_steps)
            del saved, out_s
        del bw_ws, dy

    if args.copy_bytes > 0:  # one plain copy of known size, for counter calibration
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    blas_ref = None
    if args.blas_reference and cfg.dtype == "bf16":
        blas_ref = blas_reference(cfg, int((out["counts"] - out["overflow"]).sum().item()), dev)

    ms_step = (t1 - t0) * 1e3 / args.steps
    # per-stage time of each step; the median over the steps
    stage_each = np.array([[evs[s_ - 1].elapsed_time(evs[s_]) for s_ in range(1, moe.STAGE_COUNT)]
                           for evs in events])
    stage_ms = np.median(stage_each, axis=0)

    counts = out["counts"].cpu().numpy().astype(np.int64)
    dg = out["diag"].cpu().numpy().astype(float)
    diag = {"entropy": round(dg[0], 5), "load_gini": round(dg[1], 5),
            "max_over_mean_load": round(dg[2], 4), "importance_cv2": round(dg[3], 6)}
    overflow = out["overflow"].cpu().numpy().astype(np.int64)
    kept = int((counts - overflow).sum())
    T, d, E, k, M, S = cfg.T, cfg.d, cfg.E, cfg.k, cfg.M, cfg.S
    eb = 2 if cfg.dtype == "bf16" else 4
    fl = {"gemm_up": 4.0 * d * M * kept, "gemm_down": 2.0 * d * M * kept,
          "shared": 6.0 * d * S * M * T, "route": 2.0 * d * E * T}
    # bf16 layers run their shared experts inside the routed grouped launches (a second product
    # of one group): the shared stage then reads ~0 and its flops belong to the GEMM stages
    sh_ms = float(stage_ms[moe.STAGES.index("shared")])
    shared_folded = S > 0 and sh_ms < 0.02 * float(stage_ms[moe.STAGES.index("gemm_up")])
    if shared_folded:
        fl["gemm_up"] += 4.0 * d * S * M * T
        fl["gemm_down"] += 2.0 * d * S * M * T
        fl["shared"] = 0.0
    by = {"route": T * d * eb + E * d * eb + T * k * 8,
          # placement only (indices); the gate/up GEMM gathers the x rows itself
          "dispatch": T * k * 8 + kept * 4,
          "combine": kept * d * eb + T * k * 8 + (T * d * eb if S else 0) + T * d * eb}
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    stages = {}
    for i, nm in enumerate(moe.STAGES):
        ms = float(stage_ms[i])
        st = {"ms": round(ms, 4)}
        if nm in fl and ms > 0 and fl[nm] > 0:
            tf = fl[nm] / (ms * 1e-3) / 1e12
            st.update({"tflops": round(tf, 1), "mfma_frac": round(tf / peak, 4)})
        if nm in by and ms > 0:
            gb = by[nm] / (ms * 1e-3) / 1e9
            st.update({"gbs": round(gb, 1), "hbm_frac": round(gb / PEAK_HBM_GBS, 4)})
        stages[nm] = st

    total_flops = fl["gemm_up"] + fl["gemm_down"] + fl["shared"] + fl["route"]
    layer_tf = total_flops / (ms_step * 1e-3) / 1e12
    up_ms = float(stage_ms[moe.STAGES.index("gemm_up")])
    achieved = fl["gemm_up"] / (up_ms * 1e-3) / 1e12
    traffic = load_traffic(name)
    up_each = stage_each[:, moe.STAGES.index("gemm_up")]
    roofline = {"bound": "mfma",
                "kernel": "grouped gate/up GEMM + SwiGLU (routed" +
                          (" and shared experts, one launch)" if shared_folded else ")"),
                "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "flops_per_launch": fl["gemm_up"], "ms_per_launch": round(up_ms, 4),
                "ms_per_launch_mean": round(float(up_each.mean()), 4),
                "ms_per_launch_p10_p90": [round(float(np.percentile(up_each, 10)), 4),
                                          round(float(np.percentile(up_each, 90)), 4)],
                "launches": int(args.steps)}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, host, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(T / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "step_ms": {"median": round(float(np.median(step_ms_each)), 4),
                    "p10": round(float(np.percentile(step_ms_each, 10)), 4),
                    "p90": round(float(np.percentile(step_ms_each, 90)), 4),
                    "min": round(float(step_ms_each.min()), 4),
                    "max": round(float(step_ms_each.max()), 4), "steps": int(args.steps),
                    "how": "each step between two events on the stream, a second pass"},
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": name, "T": T, "d": d, "E": E, "k": k, "M": M, "S": S,
                   "capacity_factor": cfg.c, "bias": cfg.bias, "scoring": cfg.scoring,
                   "routing": cfg.routing,
                   "kept_assignments": kept,
                   "dropped_assignments": int(overflow.sum()), "max_load": int(counts.max()),
                   "routing_diagnostics": diag},
        "mfma_peak_frac_layer": round(layer_tf / peak, 4), "layer_tflops": round(layer_tf, 1),
        "roofline": roofline, "stages": stages, "cpu_baseline": cpu,
        # router gradients of aux + z (dlogits, dW_r, dx): route in column mode + 2 fp32 GEMMs
        "balance_loss_backward": {"ms": round(lb_ms, 4),
                                  "flops": 2.0 * 3 * T * d * E},
    }
    if blas_ref is not None:
        line["blas_reference"] = blas_ref
    if bw_ms is not None:
        # algorithmic products: gate/up recompute 4dM, P = dy W_down 2dM, dx rows 4dM, weight
        # gradients 6dM per kept row; shared experts the same per token; router 2dE (logits) +
        # 4dE (dW_r, dx) per token
        bw_fl = 16.0 * d * M * kept + 16.0 * d * S * M * T + 6.0 * d * E * T
        bw_tf = bw_fl / (bw_ms * 1e-3) / 1e12
        line["layer_backward"] = {"ms": round(bw_ms, 3), "flops": bw_fl,
                                  "tflops": round(bw_tf, 1), "mfma_frac": round(bw_tf / peak, 4),
                                  "steps": args.backward_steps}
        if train_saved is not None:
            # forward + backward per training step: recomputing the gate/up pre-activations in the
            # backward, or keeping them from the forward (moe_saved_size bytes)
            line["train_step"] = {
                "recompute": {"forward_ms": round(ms_step, 4), "backward_ms": round(bw_ms, 3),
                              "total_ms": round(ms_step + bw_ms, 3)},
                "saved_pre_activations": {"forward_ms": round(train_saved[0], 4),
                                          "backward_ms": round(train_saved[1], 3),
                                          "total_ms": round(sum(train_saved), 3),
                                          "saved_bytes": moe.saved_size(layer.shape)}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
