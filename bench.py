"""Benchmark of the fused LoRA-bypass linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full forward -- operand preparation, the h contraction with its
rounding guard, and the fused main contraction with the bypass fold and the
bias/cast epilogue -- over inputs already resident in HBM.  The default
workload is the largest single-GPU one (bf16 16384x8192x8192, rank 128, bias,
log-normal rows).  W untimed steps, then K timed steps bracketed by device
synchronisation (this sets `value`), split into up to 15 blocks with events
between them (median and range), then the same K steps again with a HIP event
pair around every kernel launch for per-kernel device durations.  One JSON
line is printed with throughput (algorithmic TFLOP/s), the fraction of the
MFMA fp16/bf16 dense peak, max/RMS ULP against the fp64 oracle on sampled
rows, the roofline of the dominant kernel, the oracle's own throughput on the
host's cores, the eager two-GEMM torch chain as a comparator, and the same
figures for the other two large LoRA workloads (`large_configs`).
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

METRIC = "fused LoRA-linear TFLOP/s & % MFMA peak (fp16/bf16); max ULP vs fp64 oracle"
PEAK_TFLOPS = {1: 2500.0, 2: 2500.0, 3: 157.3}   # MI355X dense MFMA: fp16/bf16, fp32
HBM_GBS = 8000.0
# the largest single-GPU workload sets `value`; the other two large LoRA
# workloads are reported beside it (`large_configs`)
DEFAULT = "lora_bf16_16384x8192x8192_r128"
LARGE = ("lora_f16_4096x3072x3072_r16", "lora_bf16x_f32w_8192x4096x4096_r64", "lora_bf16_16384x8192x8192_r128")
AFFINE = "affine_f16_1024x768x1024"   # the plain affine configuration
BLOCKS = 15   # timed blocks (median and range), as in the Luminal page's protocol


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-eager", action="store_true")
    ap.add_argument("--no-large-configs", action="store_true", help="skip the other large LoRA workloads")
    ap.add_argument("--no-small-m", action="store_true", help="skip the small-M (decode-like) timings")
    ap.add_argument("--no-merge", action="store_true", help="skip the LoRA merge timing")
    ap.add_argument("--merge-only", action="store_true",
                    help="time only the LoRA merge of the workload's weights (profiling runs)")
    ap.add_argument("--merge-steps", type=int, default=100)
    ap.add_argument("--no-backward", action="store_true", help="skip the LoRA-bypass backward timing")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward of the workload (profiling runs)")
    ap.add_argument("--backward-steps", type=int, default=30)
    ap.add_argument("--no-dora", action="store_true", help="skip the DoRA timing")
    ap.add_argument("--dora-only", action="store_true", help="time only DoRA's norms and forward (profiling runs)")
    ap.add_argument("--dora-steps", type=int, default=50)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as WL

    wl = WL.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inputs = WL.generate(wl)
    lora = wl.kind == "lora"

    if args.merge_only or args.dora_only or args.backward_only:
        if args.copy_calibration_mib > 0:
            _copy_calibration(dev, args.copy_calibration_mib)
        if args.merge_only:
            r = {"merge": _merge(dev, wl, inputs, args.merge_steps, args.merge_steps, not args.no_cpu_baseline)}
        elif args.dora_only:
            r = {"dora": _dora(dev, wl, inputs, args.dora_steps, args.dora_steps, not args.no_cpu_baseline)}
        else:
            r = {"backward": _backward(dev, wl, inputs, args.backward_steps, args.backward_steps,
                                       not args.no_cpu_baseline, not args.no_eager)}
        print(json.dumps(dict(workload=wl.name, **r)))
        return

    if args.copy_calibration_mib > 0:
        _copy_calibration(dev, args.copy_calibration_mib)
    fb = _forward_bench(dev, wl, inputs, args.steps, args.warmup)
    c_dt, y = fb.pop("_c_dt"), fb.pop("_y")
    d = fb.pop("_d")
    out = {"metric": METRIC, "value": fb["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": fb["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": {1: "f16", 2: "bf16", 3: "f32"}[c_dt],
           "data": "synthetic (seeded Philox draws, shapes and distributions of the workload)",
           "config": {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "rank": wl.r, "scale": wl.scale,
                      "x_dtype": WL.NAME[wl.x_dt], "w_dtype": WL.NAME[wl.w_dt],
                      "bias": WL.NAME[wl.b_dt] if wl.b_dt else None, "accumulate": "f32",
                      "parallelism": "single GPU"}}
    out.update({k: v for k, v in fb.items() if k not in ("tflops", "ms_per_step")})

    # accuracy on sampled rows against the fp64 oracle; the same oracle run,
    # timed, is the CPU baseline (rank 0, one GPU)
    rows = res = None
    if not args.no_cpu_baseline:
        acc, cpu, rows, res = _accuracy(wl, inputs, y, args.cpu_seconds, timed=True)
        out.update(acc)
        out["cpu_baseline"] = cpu
        if not args.no_eager:
            out["eager_baseline"] = _eager(d, wl, c_dt, rows, res, args.steps)
    del y, d
    if lora and not args.no_large_configs:
        out["large_configs"] = {}
        for name in LARGE:
            if name == wl.name:
                continue
            w2 = WL.WORKLOADS[name]
            in2 = WL.generate(w2)
            f2 = _forward_bench(dev, w2, in2, args.steps, args.warmup)
            c2, y2, d2 = f2.pop("_c_dt"), f2.pop("_y"), f2.pop("_d")
            for k in ("input_digest", "instrumented_ms_per_step"):
                f2.pop(k, None)
            if not args.no_cpu_baseline:
                acc2, _, rows2, res2 = _accuracy(w2, in2, y2, 4.0, timed=False)
                f2.update(acc2)
                if not args.no_eager:
                    f2["eager_baseline"] = _eager(d2, w2, c2, rows2, res2, args.steps)
            if w2.w_dt == WL.F32 and c2 != WL.F32:
                # fp32 master weights: the same forward with their bf16 copy kept
                f2["with_kept_compute_copy"] = _kept_copy_bench(dev, w2, in2, args.steps, args.warmup)
            out["large_configs"][name] = f2
            del y2, d2, in2
            torch.cuda.empty_cache()

    if lora and not args.no_large_configs:
        # the plain affine configuration, and the same with W prepared once
        wa = WL.WORKLOADS[AFFINE]
        ina = WL.generate(wa)
        fa = _forward_bench(dev, wa, ina, args.steps, args.warmup)
        ya = fa.pop("_y")
        for k in ("_c_dt", "_d", "input_digest", "instrumented_ms_per_step"):
            fa.pop(k, None)
        if not args.no_cpu_baseline:
            acca, _, _, _ = _accuracy(wa, ina, ya, 2.0, timed=False)
            fa.update(acca)
        fa["with_prepared_weight"] = _prepared_affine_bench(dev, wa, ina, args.steps, args.warmup)
        out["affine"] = fa
        del ya, ina
        torch.cuda.empty_cache()
    elif not lora:
        out["with_prepared_weight"] = _prepared_affine_bench(dev, wl, inputs, args.steps, args.warmup)

    # the tile planner's device model, measured on this GPU (its shortlist
    # order in small_m[].tuned follows these rates)
    import lora_bypass_linear_amd as L
    rates = L.measure_device_rates(dev)
    out["device_rates"] = {"cus": rates["cus"], "mfma16_tflops": round(rates["mfma16_flops"] / 1e12, 1),
                           "mfma32_tflops": round(rates["mfma32_flops"] / 1e12, 1),
                           "hbm_copy_gbs": round(rates["hbm_bytes_per_s"] / 1e9, 1)}
    if not args.no_small_m:
        out["small_m"] = _small_m(dev)
    if lora and wl.r > 0 and not args.no_merge:
        out["merge"] = _merge(dev, wl, inputs, args.merge_steps, 20, not args.no_cpu_baseline)
    if lora and wl.r > 0 and not args.no_dora:
        out["dora"] = _dora(dev, wl, inputs, args.dora_steps, 10, not args.no_cpu_baseline)
    if lora and wl.r > 0 and not args.no_backward:
        out["backward"] = _backward(dev, wl, inputs, args.backward_steps, 10, not args.no_cpu_baseline,
                                    not args.no_eager)
    print(json.dumps(out))


def _kept_copy_bench(dev, wl, inputs, steps, warmup):
    """The forward of an fp32-weight workload with W's compute-dtype copy kept
    by the caller (made once, not cast per call): wall time per step over K
    steps after W warm-up steps, and each kernel kind's device time."""
    import torch

    import lora_bypass_linear_amd as L

    d = {k: v.to(dev) for k, v in inputs.items()}
    dts = [L.dtype_code(d[k]) for k in ("x", "w", "down", "up")] + ([L.dtype_code(d["b"])] if "b" in d else [])
    c_dt, o_dt = L.resolve_dtypes(dts)
    w_c = d["w"].to(L.torch_dtype(c_dt)).contiguous()
    y, ws = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), return_workspace=True, w_c=w_c)
    step = lambda: L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), out=y, workspace=ws,
                                 w_c=w_c)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    L.profile_begin(8 * steps)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = L.profile_end()
    return {"ms_per_step": round(ms, 5), "tflops": round(wl.flops / (ms * 1e-3) / 1e12, 2),
            "kernels": {k: {"launches": n, "avg_us": round(t * 1e3 / max(n, 1), 3)} for k, (n, t) in prof.items()
                        if n}}


def _prepared_affine_bench(dev, wl, inputs, steps, warmup):
    """The plain affine forward with W prepared once (its split kept in the
    workspace by the caller): wall time per step over K steps after W warm-up
    steps, and each kernel kind's device time."""
    import torch

    import lora_bypass_linear_amd as L

    d = {k: v.to(dev) for k, v in inputs.items()}
    x, w, b = d["x"], d["w"], d.get("b")
    ws = L.linear_prepare(w, wl.M, x.dtype, b.dtype if b is not None else None)
    y = L.linear(x, w, b, workspace=ws, prepared=True)
    step = lambda: L.linear(x, w, b, out=y, workspace=ws, prepared=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    L.profile_begin(8 * steps)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = L.profile_end()
    return {"ms_per_step": round(ms, 5), "tflops": round(wl.flops / (ms * 1e-3) / 1e12, 2),
            "kernels": {k: {"launches": n, "avg_us": round(t * 1e3 / max(n, 1), 3)} for k, (n, t) in prof.items()
                        if n}}


def _forward_bench(dev, wl, inputs, steps, warmup):
    """One workload's forward: W untimed steps, then K timed steps bracketed by
    device synchronisation (wall clock: `tflops`, `ms_per_step`), split into
    up to 15 blocks with events on the launch stream between them (median and
    range per step); then the same K steps with a HIP event pair around every
    kernel launch (per-kernel device durations; the dominant kernel's
    roofline).  Returns a dict (plus the output and device inputs under
    private keys)."""
    import torch

    import lora_bypass_linear_amd as L
    import workloads as WL

    d = {k: v.to(dev) for k, v in inputs.items()}
    lora = wl.kind == "lora"
    b_dt = L.dtype_code(d["b"]) if "b" in d else 0
    dts = [L.dtype_code(d["x"]), L.dtype_code(d["w"])] + ([b_dt] if b_dt else []) + \
          ([L.dtype_code(d["down"]), L.dtype_code(d["up"])] if lora else [])
    c_dt, o_dt = L.resolve_dtypes(dts)
    y = torch.empty((wl.M, wl.N), dtype=L.torch_dtype(o_dt), device=dev)
    if lora:
        nws = L.lora_workspace_size(wl.M, wl.N, wl.K, wl.r, dts[0], dts[1], b_dt, L.dtype_code(d["down"]),
                                    L.dtype_code(d["up"]))
    else:
        nws = L.linear_workspace_size(wl.M, wl.N, wl.K, dts[0], dts[1], b_dt)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        if lora:
            L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), out=y, workspace=ws)
        else:
            L.linear(d["x"], d["w"], d.get("b"), out=y, workspace=ws)

    print(f"[bench] {wl.name}: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, nothing else on the stream but the block events
    nb = max(1, min(BLOCKS, steps))
    sizes = [steps // nb + (1 if i < steps % nb else 0) for i in range(nb)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    print(f"[bench] timing {steps} steps in {nb} blocks", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i, n in enumerate(sizes):
        for _ in range(n):
            step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    per_block = sorted(ev[i].elapsed_time(ev[i + 1]) / sizes[i] for i in range(nb) if sizes[i] > 0)
    med = per_block[len(per_block) // 2] if len(per_block) % 2 else \
        0.5 * (per_block[len(per_block) // 2 - 1] + per_block[len(per_block) // 2])

    # the same K steps again with a HIP event pair around every kernel launch,
    # on the launch stream, for per-kernel device durations (the event records
    # add gaps between kernels, so this region sets neither value nor blocks)
    print(f"[bench] timing {steps} instrumented steps", file=sys.stderr, flush=True)
    L.profile_begin(8 * steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_i = time.perf_counter() - t0
    prof = L.profile_end()

    # dominant kernel: the fused main contraction (fold + K loop + epilogue) of
    # the LoRA path, or the plain affine path's contraction (recorded as the
    # GEMM kind)
    dom = "gemm" if lora else "hpass"
    n_g, t_g = prof["gemm"]
    dom_ms = t_g / max(n_g, 1)
    dom_flops = 2.0 * wl.M * wl.N * wl.K + (2.0 * wl.M * wl.r * wl.N if lora else 0.0)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12 if dom_ms > 0 else 0.0
    peak = PEAK_TFLOPS[c_dt]
    from lora_bypass_linear_amd.profsum import read_traffic
    traffic = read_traffic(os.path.join(ROOT, "profiles", f"traffic_{dom}_{wl.name}.txt"), dom)
    tflops = wl.flops / (ms_per_step * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "gemm_kernel" if lora else "xr_kernel", "achieved": round(achieved, 2),
                "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None if traffic is None else int(traffic),
                "flops_per_launch": dom_flops, "avg_us": round(dom_ms * 1e3, 3)}
    kernels = {k: {"launches": n, "avg_us": round(t * 1e3 / n, 3)} for k, (n, t) in prof.items() if n}
    guard = None
    if lora and wl.r > 0 and c_dt != L.F32:
        _, _, fo, ns = L.lora_workspace_layout(wl.M, wl.N, wl.K, wl.r, dts[0], dts[1], b_dt,
                                               L.dtype_code(d["down"]), L.dtype_code(d["up"]))
        nflag = int(ws[fo: fo + 4 * ns].cpu().view(torch.int32).sum().item())
        guard = {"h_reevaluated_fp64": nflag, "of": wl.M * wl.r, "fraction": round(nflag / (wl.M * wl.r), 6)}
    elif not lora and c_dt != L.F32:
        fo, ns = L.linear_workspace_layout(wl.M, wl.N, wl.K, dts[0], dts[1], b_dt)
        nflag = int(ws[fo: fo + 4 * ns].cpu().view(torch.int32).sum().item())
        guard = {"projection_reevaluated_fp64": nflag, "of": wl.M * wl.N,
                 "fraction": round(nflag / (wl.M * wl.N), 6)}
    return {"tflops": round(tflops, 2), "ms_per_step": round(ms_per_step, 5),
            "blocks": {"n": nb, "steps_per_block": sizes, "median_ms_per_step": round(med, 5),
                       "min_ms_per_step": round(per_block[0], 5), "max_ms_per_step": round(per_block[-1], 5),
                       "median_tflops": round(wl.flops / (med * 1e-3) / 1e12, 2)},
            "frac_of_peak": round(tflops / peak, 4), "hbm_gbs": round(wl.bytes / (ms_per_step * 1e-3) / 1e9, 1),
            "instrumented_ms_per_step": round(wall_i * 1e3 / steps, 5), "input_digest": WL.digest(inputs),
            "kernels": kernels, "h_guard": guard, "roofline": roofline,
            "_c_dt": c_dt, "_y": y, "_d": d}


def _accuracy(wl, inputs, y, cpu_seconds, timed):
    """Max/RMS ULP and the per-element tolerance on sampled output rows against
    the fp64 oracle, which runs on every host CPU this process may use.  With
    `timed`, the sample is sized from two timed probes (a call costs a fixed
    part, widening every operand, plus a part per output row) to about
    `cpu_seconds` of oracle work, and the oracle's throughput is returned as
    the CPU baseline."""
    import numpy as np

    import oracle
    import workloads as WL
    from tests.gpu_cases import score

    bits = {k: WL.raw_bits(v) for k, v in inputs.items()}
    dt = {k: WL.dtype_code(v) for k, v in inputs.items()}
    cores, aff, quota = oracle.host_cpus()

    def run(rows):
        return oracle.forward(bits["x"], dt["x"], bits["w"], dt["w"], bits.get("b"), dt.get("b"), bits.get("down"),
                              dt.get("down"), bits.get("up"), dt.get("up"), scale=wl.scale, rows=rows,
                              nthreads=cores, lora=wl.kind == "lora")

    y_cpu = y.cpu()
    rng = np.random.default_rng(wl.seed)
    probe_rows = np.sort(rng.choice(wl.M, size=min(wl.M, 4 * cores), replace=False))
    small = probe_rows[: max(1, probe_rows.size // 4)]
    run(small)
    t1 = time.perf_counter()
    run(small)
    t_small = time.perf_counter() - t1
    t1 = time.perf_counter()
    run(probe_rows)
    t_big = time.perf_counter() - t1
    per_row = max((t_big - t_small) / max(probe_rows.size - small.size, 1), 1e-6)
    fixed = max(t_small - per_row * small.size, 0.0)
    want_rows = max(cpu_seconds - fixed, per_row) / per_row
    n_rows = int(min(wl.M, max(cores, want_rows)))
    # a workload whose every row fits in the budget is passed over whole, several times
    passes = int(max(1, min(20, round(cpu_seconds / (fixed + per_row * wl.M))))) if (timed and n_rows == wl.M) else 1
    rows = np.sort(rng.choice(wl.M, size=n_rows, replace=False))
    print(f"[bench] oracle on {n_rows} rows x {passes}, {cores} threads", file=sys.stderr, flush=True)
    t1 = time.perf_counter()
    for _ in range(passes):
        res = run(rows)
    t_cpu = time.perf_counter() - t1
    s = score(y_cpu, res, rows, wl.K, wl.r)
    acc = {"max_ulp": round(s["ulp_max"], 4), "rms_ulp": round(s["ulp_rms"], 4), "tol_fail": s["fail"],
           "tol_checked": s["n"], "worst_err_over_tol": round(s["worst"], 4), "rows_checked": int(n_rows)}
    cpu = None
    if timed:
        row_flops = wl.flops / wl.M
        cpu = {"value": round(row_flops * n_rows * passes / t_cpu / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
               "cores_affinity": aff, "cpu_quota": quota, "kind": "oracle",
               "sample": f"{n_rows} of {wl.M} output rows (all {wl.N} columns)"
                         + (f", {passes} passes" if passes > 1 else "") + f", {t_cpu:.1f} s"}
    return acc, cpu, rows, res


def _copy_calibration(dev, mib):
    """One plain device copy of a known size (scales the HBM byte counters)."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _merge(dev, wl, inputs, reps, warm, accuracy):
    """The LoRA merge W' = round_out(W + scale * up_c.down_c) of the workload's
    weights (out of place): wall and device time per call, algorithmic HBM
    bytes (read W, down, up; write W') over the merge contraction's device time
    against the 8 TB/s peak, and, on sampled rows, ULP against the fp64 oracle
    next to the eager torch chain (up.down rounded to the compute dtype, then
    scaled and added to W, each step rounding)."""
    import numpy as np
    import torch

    import lora_bypass_linear_amd as L
    import workloads as WL

    w, dn, up = (inputs[k].to(dev) for k in ("w", "down", "up"))
    dts = [L.dtype_code(w), L.dtype_code(dn), L.dtype_code(up)]
    c_dt, o_dt = L.resolve_dtypes(dts)
    out = torch.empty((wl.N, wl.K), dtype=L.torch_dtype(o_dt), device=dev)
    nws = L.lora_merge_workspace_size(wl.N, wl.K, wl.r, *dts)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    call = lambda: L.lora_merge(w, dn, up, wl.scale, out=out, workspace=ws)
    print(f"[bench] merge {wl.name}: {warm} + {reps} calls", file=sys.stderr, flush=True)
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) * 1e6 / reps
    L.profile_begin(4 * reps)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    prof = L.profile_end()
    es = {L.F16: 2, L.BF16: 2, L.F32: 4}
    nbytes = wl.N * wl.K * (es[dts[0]] + es[o_dt]) + wl.r * wl.K * es[dts[1]] + wl.N * wl.r * es[dts[2]]
    n_g, t_g = prof["gemm"]
    g_us = t_g * 1e3 / max(n_g, 1)
    dev_us = sum(ms for _, ms in prof.values()) * 1e3 / reps
    from lora_bypass_linear_amd.profsum import read_traffic
    traffic = read_traffic(os.path.join(ROOT, "profiles", f"traffic_merge_{wl.name}.txt"), "merge")
    kname = _merge_kernel_name(c_dt, dts[0], dts[1], dts[2], o_dt, wl.K, wl.r)
    r = {"shape": f"W [{wl.N},{wl.K}] {WL.NAME[wl.w_dt]}, rank {wl.r}, scale {wl.scale}",
         "wall_us_per_call": round(wall_us, 2), "device_us_per_call": round(dev_us, 2),
         "kernels": {{"prep": "merge_prep_kernel", "gemm": kname}.get(k, k):
                     {"launches": n, "avg_us": round(ms * 1e3 / n, 3)} for k, (n, ms) in prof.items() if n},
         "hbm_gbs_call": round(nbytes / (dev_us * 1e-6) / 1e9, 1),
         "roofline": _stream_roofline(kname, nbytes, 2 * wl.N * wl.K * wl.r, c_dt, g_us, traffic)}
    if accuracy:
        import oracle
        from tests.gpu_cases import sample_rows, score
        rows = sample_rows(wl.N, 32, seed=wl.seed, tile=128)
        res = oracle.merge(WL.raw_bits(inputs["w"]), dts[0], WL.raw_bits(inputs["down"]), dts[1],
                           WL.raw_bits(inputs["up"]), dts[2], scale=wl.scale, rows=rows)
        s = score(out.cpu(), res, rows, wl.r, 0)
        ct, ot = L.torch_dtype(c_dt), L.torch_dtype(o_dt)
        delta = torch.matmul(up.to(ct), dn.to(ct).contiguous())
        eager = (w.to(ot) + (delta * wl.scale).to(ot)).to(ot) if o_dt == L.F32 else (w + delta * wl.scale).to(ot)
        torch.cuda.synchronize()
        se = score(eager.cpu(), res, rows, wl.r, 0)
        r.update({"rows_checked": int(np.asarray(rows).size), "max_ulp": round(s["ulp_max"], 4),
                  "rms_ulp": round(s["ulp_rms"], 4), "tol_fail": s["fail"],
                  "eager": {"max_ulp": round(se["ulp_max"], 4), "rms_ulp": round(se["ulp_rms"], 4),
                            "tol_fail": se["fail"]}})
    return r


def _stream_roofline(kname, nbytes, flops, c_dt, avg_us, traffic):
    """Roofline of a merge or row-norm launch: whichever of its HBM bytes at
    8 TB/s and its contraction at the compute dtype's MFMA peak takes longer
    is the bound (the fp32 contraction at 157.3 TFLOP/s can take longer than
    the weight's stream)."""
    hbm_us = nbytes / (HBM_GBS * 1e9) * 1e6
    mfma_us = flops / (PEAK_TFLOPS[c_dt] * 1e12) * 1e6
    floors = {"hbm_floor_us": round(hbm_us, 3), "mfma_floor_us": round(mfma_us, 3)}
    if mfma_us > hbm_us:
        ach = flops / (avg_us * 1e-6) / 1e12
        return {"bound": "mfma", "kernel": kname, "achieved": round(ach, 2), "peak": PEAK_TFLOPS[c_dt],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[c_dt], 4),
                "traffic": None if traffic is None else int(traffic), "bytes_per_launch": nbytes,
                "flops_per_launch": flops, "avg_us": round(avg_us, 3), **floors}
    ach = nbytes / (avg_us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1), "peak": HBM_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_GBS, 4), "traffic": None if traffic is None else int(traffic),
            "bytes_per_launch": nbytes, "flops_per_launch": flops, "avg_us": round(avg_us, 3), **floors}


def _merge_kernel_name(c_dt, w_dt, d_dt, u_dt, o_dt, K, r):
    """The merge kernel the library launches for these dtypes and sizes: the
    streaming form takes 16-bit compute with W, W' and both factors in it (read
    as stored, so rank and K multiples of 8) and a padded rank up to 128."""
    import lora_bypass_linear_amd as L
    half = c_dt in (L.F16, L.BF16) and w_dt == c_dt and o_dt == c_dt and d_dt == c_dt and u_dt == c_dt
    return "merge_stream_kernel" if half and K % 8 == 0 and r % 8 == 0 and 0 < r <= 128 else "merge_kernel"


def _dora(dev, wl, inputs, reps, warm, accuracy):
    """DoRA: the row norms of the merged weight (device time, HBM bytes of W,
    down and up read and the norms written, against 8 TB/s) and the DoRA
    forward beside the plain LoRA forward of the same shape (the gain's
    cost), with ULP against the fp64 oracle on sampled rows."""
    import numpy as np
    import torch

    import lora_bypass_linear_amd as L
    import workloads as WL

    d = {k: v.to(dev) for k, v in inputs.items()}
    mag = WL.generate_magnitude(wl)
    m = mag.to(dev)
    norms = torch.empty(wl.N, dtype=torch.float32, device=dev)
    print(f"[bench] dora {wl.name}: {warm} + {reps} calls", file=sys.stderr, flush=True)

    def timed_calls(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e6 / reps
        L.profile_begin(8 * reps)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return wall, L.profile_end()

    nfn = lambda: L.dora_norms(d["w"], d["down"], d["up"], wl.scale, out=norms)
    wall_n, prof_n = timed_calls(nfn)
    es = {L.F16: 2, L.BF16: 2, L.F32: 4}
    w_dt, d_dt, u_dt = (L.dtype_code(d[k]) for k in ("w", "down", "up"))
    nbytes = wl.N * wl.K * es[w_dt] + wl.r * wl.K * es[d_dt] + wl.N * wl.r * es[u_dt] + wl.N * 4
    n_g, t_g = prof_n["gemm"]
    g_us = t_g * 1e3 / max(n_g, 1)
    c_dt, o_dt = L.resolve_dtypes([w_dt, d_dt, u_dt])
    kname = _merge_kernel_name(c_dt, w_dt, d_dt, u_dt, c_dt, wl.K, wl.r)
    y = L.dora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, m, norms, d.get("b"))
    wall_f, prof_f = timed_calls(lambda: L.dora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, m, norms,
                                                       d.get("b"), out=y))
    yl = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"))
    wall_l, prof_l = timed_calls(lambda: L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"),
                                                       out=yl))
    dev_us = lambda prof: round(sum(ms for _, ms in prof.values()) * 1e3 / reps, 2)
    # the norm pass's HBM bytes from its counter profile (null once its sources changed)
    from lora_bypass_linear_amd.profsum import read_traffic
    traffic = read_traffic(os.path.join(ROOT, "profiles", f"traffic_doranorm_{wl.name}.txt"), "merge")
    out = {"shape": f"M {wl.M}, N {wl.N}, K {wl.K}, rank {wl.r}, magnitude {WL.NAME[L.dtype_code(m)]}",
           "norms": {"wall_us_per_call": round(wall_n, 2), "device_us_per_call": dev_us(prof_n),
                     "roofline": _stream_roofline(kname + " (row norms)", nbytes, 2 * wl.N * wl.K * wl.r,
                                                  c_dt, g_us, traffic)},
           "forward": {"wall_us_per_call": round(wall_f, 2), "device_us_per_call": dev_us(prof_f),
                       "tflops": round(wl.flops / (dev_us(prof_f) * 1e-6) / 1e12, 2),
                       "lora_forward_device_us": dev_us(prof_l)}}
    if accuracy:
        import oracle
        from tests.gpu_cases import sample_rows, score
        rows = sample_rows(wl.M, 24, seed=wl.seed)
        bits = {k: WL.raw_bits(v) for k, v in inputs.items()}
        dt = {k: WL.dtype_code(v) for k, v in inputs.items()}
        res = oracle.dora_forward(bits["x"], dt["x"], bits["w"], dt["w"], bits.get("b"), dt.get("b"), bits["down"],
                                  dt["down"], bits["up"], dt["up"], WL.raw_bits(mag), WL.dtype_code(mag),
                                  scale=wl.scale, rows=rows)
        sc = score(y.cpu(), res, rows, wl.K, wl.r)
        nrel = np.abs(norms.cpu().numpy().astype(np.float64) - res["norms"].astype(np.float64)) / res["norms"]
        out["forward"].update({"max_ulp": round(sc["ulp_max"], 4), "rms_ulp": round(sc["ulp_rms"], 4),
                               "tol_fail": sc["fail"], "rows_checked": int(len(rows))})
        out["norms"]["max_rel_err_vs_oracle"] = float(nrel.max())
    return out


def _backward(dev, wl, inputs, reps, warm, accuracy, eager):
    """The LoRA-bypass backward for a seeded dy (N(0,1) in the forward's output
    dtype): wall time per call with all three gradients, the device time of
    each kernel kind, algorithmic TFLOP/s, and the dx GEMM's roofline from a
    dx-only call (its GEMM launch alone); on sampled rows / columns / rank
    indices, ULP against the fp64 oracle next to the eager torch autograd
    chain."""
    import numpy as np
    import torch

    import lora_bypass_linear_amd as L
    import workloads as WL

    M, N, K, r = wl.M, wl.N, wl.K, wl.r
    d = {k: v.to(dev) for k, v in inputs.items()}
    codes = [WL.dtype_code(inputs[k]) for k in ("x", "w", "down", "up")] + \
            ([WL.dtype_code(inputs["b"])] if "b" in inputs else [])
    c_dt, o_dt = L.resolve_dtypes(codes)
    dy_cpu = WL.generate_dy(wl, o_dt)
    dy = dy_cpu.to(dev)
    b_dtype = inputs["b"].dtype if "b" in inputs else None
    ws = torch.empty(max(L.lora_bwd_workspace_size(M, N, K, r, codes[0], codes[1], WL.dtype_code(inputs["b"])
                                                   if "b" in inputs else 0, codes[2], codes[3],
                                                   WL.dtype_code(dy_cpu), 7), 1), dtype=torch.uint8, device=dev)
    call = lambda **kw: L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], wl.scale, dy, bias_dtype=b_dtype,
                                               workspace=ws, **kw)
    print(f"[bench] backward {wl.name}: {warm} + {reps} calls", file=sys.stderr, flush=True)
    for _ in range(warm):
        grads = call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        grads = call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    L.profile_begin(32 * reps)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    prof = L.profile_end()
    # dx alone: its one GEMM launch is the dominant kernel of the backward
    for _ in range(5):
        call(want_ddown=False, want_dup=False)
    L.profile_begin(16 * reps)
    for _ in range(reps):
        call(want_ddown=False, want_dup=False)
    torch.cuda.synchronize()
    pdx = L.profile_end()
    n_g, t_g = pdx["gemm"]
    g_us = t_g * 1e3 / max(n_g, 1)
    dx_flops = 2.0 * M * N * K + 2.0 * M * r * K
    flops = 2.0 * M * K * r + 2.0 * M * N * r + dx_flops + 2.0 * M * r * K + 2.0 * M * N * r
    peak = PEAK_TFLOPS[c_dt]
    names = {"cast": "transposes + casts", "prep": "prep + row norms", "hpass": "h and gh passes",
             "gemm": "dx, dDown, dUp GEMMs"}
    # the same calls with a caller-kept W_c^T (W frozen across steps): no W^T copy per call
    w_t = d["w"].to(L.torch_dtype(c_dt)).t().contiguous()
    for _ in range(3):
        call(w_t=w_t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        call(w_t=w_t)
    torch.cuda.synchronize()
    ms_wt = (time.perf_counter() - t0) * 1e3 / reps
    L.profile_begin(32 * reps)
    for _ in range(reps):
        call(w_t=w_t)
    torch.cuda.synchronize()
    prof_wt = L.profile_end()
    # ... and with the h_r its forward left as well (what a training step keeps): no h pass
    _, fws = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), return_workspace=True)
    h = L.lora_saved_h(fws, d["x"], d["w"], d["down"], d["up"], d.get("b"))
    for _ in range(3):
        call(w_t=w_t, h=h)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        call(w_t=w_t, h=h)
    torch.cuda.synchronize()
    ms_st = (time.perf_counter() - t0) * 1e3 / reps
    L.profile_begin(32 * reps)
    for _ in range(reps):
        call(w_t=w_t, h=h)
    torch.cuda.synchronize()
    prof_st = L.profile_end()
    del w_t, h, fws
    out = {"shape": f"M {M}, N {N}, K {K}, rank {r}, dy {WL.NAME[WL.dtype_code(dy_cpu)]}",
           "ms_per_call": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "flops_per_call": flops,
           "kernels": {names[k]: {"launches": n // reps, "us_per_call": round(t * 1e3 / reps, 2)}
                       for k, (n, t) in prof.items() if n},
           "with_caller_wt": {"ms_per_call": round(ms_wt, 4), "tflops": round(flops / (ms_wt * 1e-3) / 1e12, 2),
                              "kernels": {names[k]: {"launches": n // reps, "us_per_call": round(t * 1e3 / reps, 2)}
                                          for k, (n, t) in prof_wt.items() if n}},
           "with_caller_wt_and_saved_h": {
               "ms_per_call": round(ms_st, 4), "tflops": round(flops / (ms_st * 1e-3) / 1e12, 2),
               "kernels": {names[k]: {"launches": n // reps, "us_per_call": round(t * 1e3 / reps, 2)}
                           for k, (n, t) in prof_st.items() if n}},
           "roofline": {"bound": "mfma", "kernel": "gemm_kernel (dx = dy_c.W_c + gh_r.down_c)",
                        "achieved": round(dx_flops / (g_us * 1e-6) / 1e12, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(dx_flops / (g_us * 1e-6) / 1e12 / peak, 4), "traffic": None,
                        "flops_per_launch": dx_flops, "avg_us": round(g_us, 3)}}
    if accuracy:
        import oracle
        from tests.gpu_cases import sample_rows
        rng = np.random.default_rng(wl.seed)
        rows = sample_rows(M, 16, seed=wl.seed)
        js = np.sort(rng.choice(r, min(r, 4), replace=False))
        kk = sample_rows(K, 24, seed=wl.seed + 1)
        nn = sample_rows(N, 24, seed=wl.seed + 2)
        bits = {k: WL.raw_bits(v) for k, v in inputs.items()}
        res = oracle.backward(bits["x"], codes[0], bits["w"], codes[1], bits["down"], codes[2], bits["up"], codes[3],
                              WL.raw_bits(dy_cpu), WL.dtype_code(dy_cpu), scale=wl.scale,
                              b_dt=WL.dtype_code(inputs["b"]) if "b" in inputs else 0, dx_rows=rows, js=js,
                              dd_cols=kk, du_rows=nn)

        def score(gx, gd, gu):
            o = {}
            for name, g, want, ref, rss, dt, length in (
                    ("dx", WL.raw_bits(gx.cpu())[rows], res["dx"], res["dx_ref"], res["dx_rss"], codes[0], N + r),
                    ("d_down", WL.raw_bits(gd.cpu())[np.ix_(js, kk)], res["d_down"], res["dd_ref"], res["dd_rss"],
                     codes[2], M),
                    ("d_up", WL.raw_bits(gu.cpu())[np.ix_(nn, js)], res["d_up"], res["du_ref"], res["du_rss"],
                     codes[3], M)):
                gv, wv = oracle.as_float64(g, dt), oracle.as_float64(want, dt)
                tol = oracle.tolerance_sum(wv, rss, c_dt, length)
                umax, urms = oracle.ulp_report(gv, ref, c_dt)
                o[name] = {"max_ulp": round(umax, 3), "rms_ulp": round(urms, 3),
                           "tol_fail": int((~((gv == wv) | (np.abs(gv - wv) <= tol))).sum()), "n": int(gv.size)}
            return o

        out["accuracy"] = score(*grads)
        if eager:
            ct = L.torch_dtype(c_dt)
            xe = d["x"].detach().clone().requires_grad_(True)
            de = d["down"].detach().clone().requires_grad_(True)
            ue = d["up"].detach().clone().requires_grad_(True)
            import torch.nn.functional as F

            def run():
                h = F.linear(xe.to(ct), de.to(ct))
                y = F.linear(xe.to(ct), d["w"].to(ct)) + wl.scale * F.linear(h, ue.to(ct))
                return torch.autograd.grad(y, (xe, de, ue), dy.to(ct))

            run()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            n = max(5, reps // 2)
            for _ in range(n):
                ge = run()
            torch.cuda.synchronize()
            ems = (time.perf_counter() - t0) * 1e3 / n
            out["eager"] = {"ms_per_call": round(ems, 4), "tflops": round(flops / (ems * 1e-3) / 1e12, 2),
                            "accuracy": score(*ge)}
    return out


def _small_m(dev, reps=50):
    """Few-token calls of config 1's plain affine shape and of the fp16 LoRA
    shape: wall time per back-to-back call (host launch cost included), the
    summed device time of the kernels of one call (HIP events), and the
    algorithmic HBM GB/s and TFLOP/s over that device time."""
    import torch

    import lora_bypass_linear_amd as L
    import workloads as WL

    res = []
    for base in ("affine_f16_1024x768x1024", "lora_f16_4096x3072x3072_r16"):
        for M in (16, 128):
            wl = WL.WORKLOADS[base].resized(M=M)
            d = {k: v.to(dev) for k, v in WL.generate(wl).items()}
            if wl.kind == "lora":
                y, ws = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), return_workspace=True)
                call = lambda: L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), out=y,
                                             workspace=ws)
            else:
                y = L.linear(d["x"], d["w"], d.get("b"))
                nb = L.linear_workspace_size(wl.M, wl.N, wl.K, L.dtype_code(d["x"]), L.dtype_code(d["w"]),
                                             L.dtype_code(d["b"]) if "b" in d else 0)
                ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
                call = lambda: L.linear(d["x"], d["w"], d.get("b"), out=y, workspace=ws)
            for _ in range(5):
                call()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                call()
            torch.cuda.synchronize()
            wall_us = (time.perf_counter() - t0) * 1e6 / reps
            L.profile_begin(8 * reps)
            for _ in range(reps):
                call()
            torch.cuda.synchronize()
            prof = L.profile_end()
            dev_us = sum(ms for _, ms in prof.values()) * 1e3 / reps
            entry = {"workload": f"{base} at M={M}", "wall_us_per_call": round(wall_us, 2),
                     "device_us_per_call": round(dev_us, 2),
                     "kernels": {k: round(ms * 1e3 / reps, 2) for k, (n, ms) in prof.items() if n},
                     "hbm_gbs": round(wl.bytes / (dev_us * 1e-6) / 1e9, 1),
                     "tflops": round(wl.flops / (dev_us * 1e-6) / 1e12, 3)}
            if wl.kind == "lora":
                # the measured tile pick: the planner's shortlist timed, then the same calls again
                c_dt = L.resolve_dtypes([L.dtype_code(d[k]) for k in ("x", "w", "down", "up")])[0]
                plan = L.gemm_plan(wl.M, wl.N, wl.K, 16, c_dt)
                tn, tm, ks, _, cand = L.lora_linear_tune(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"),
                                                         out=y, workspace=ws)
                L.profile_begin(8 * reps)
                for _ in range(reps):
                    call()
                torch.cuda.synchronize()
                tuned_us = sum(ms for _, ms in L.profile_end().values()) * 1e3 / reps
                entry["tuned"] = {"analytic_pick": list(plan[0][:3]), "pick": [tn, tm, ks],
                                  "device_us_per_call": round(tuned_us, 2),
                                  "shortlist": [{"tile": f"{p[0]}x{p[1]}", "ksplit": p[2],
                                                 "model_us": round(p[3], 2), "measured_us": round(c * 1e3, 2)}
                                                for p, c in zip(plan, cand)]}
                L.tuning_clear()
            res.append(entry)
    return res


def _eager(d, wl, c_dt, rows, res, steps):
    """The unfused torch chain, each op rounding to the compute dtype, then cast
    to the output dtype (comparator only): time per call and its ULP against
    the fp64 oracle on the same sampled rows."""
    import torch
    import torch.nn.functional as F

    import lora_bypass_linear_amd as L
    from tests.gpu_cases import score

    ct = L.torch_dtype(c_dt)
    ot = L.torch_dtype(res["output"])

    def run():
        x = d["x"].to(ct)
        w = d["w"].to(ct)
        if wl.kind == "lora":
            h = F.linear(x, d["down"].to(ct))
            yv = F.linear(x, w) + wl.scale * F.linear(h, d["up"].to(ct))
        else:
            yv = F.linear(x, w)
        if "b" in d:
            yv = yv + d["b"].to(ct)
        return yv.to(ot)

    for _ in range(3):
        yv = run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = max(5, steps // 2)
    for _ in range(n):
        yv = run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    s = score(yv.cpu(), res, rows, wl.K, wl.r)
    return {"ms_per_step": round(ms, 5), "tflops": round(wl.flops / (ms * 1e-3) / 1e12, 2),
            "max_ulp": round(s["ulp_max"], 4), "rms_ulp": round(s["ulp_rms"], 4), "tol_fail": s["fail"]}


if __name__ == "__main__":
    main()
