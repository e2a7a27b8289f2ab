"""Shared helpers for the GPU parity tests: run a workload through the C-ABI
library and through the oracle on the same seeded inputs, and score the
difference element by element."""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch

import lora_bypass_linear_amd as L
import oracle
import workloads as WL


def say(*a):
    """Name the case before each GPU step (flushed, so it survives a lost box)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def gpu_forward(inputs: Dict[str, torch.Tensor], wl: WL.Workload, scale: Optional[float] = None):
    """Run the library on `inputs` (CPU tensors).  Returns (y cpu tensor,
    h_r [M, r] float64 or None, flagged count or None)."""
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inputs.items()}
    say(wl.name, f"M={wl.M} N={wl.N} K={wl.K} r={wl.r} kind={wl.kind}")
    if wl.kind == "lora":
        s = wl.scale if scale is None else scale
        y, ws = L.lora_linear(d["x"], d["w"], d["down"], d["up"], s, d.get("b"), return_workspace=True)
        torch.cuda.synchronize()
        h = flagged = None
        if ws is not None and wl.r > 0:
            args = (wl.M, wl.N, wl.K, wl.r, L.dtype_code(d["x"]), L.dtype_code(d["w"]),
                    L.dtype_code(d["b"]) if "b" in d else 0, L.dtype_code(d["down"]), L.dtype_code(d["up"]))
            c_dt, _ = L.resolve_dtypes([a for a in (args[4], args[5], args[6], args[7], args[8]) if a])
            ho, ld, fo, ns = L.lora_workspace_layout(*args)
            es = 4 if c_dt == L.F32 else 2
            raw = ws[ho: ho + wl.M * ld * es].cpu()
            if c_dt == L.F32:
                hv = raw.view(torch.float32).numpy().reshape(wl.M, ld).astype(np.float64)
            else:
                hv = oracle.as_float64(raw.view(torch.int16).numpy().view(np.uint16).reshape(wl.M, ld), c_dt)
            h = hv[:, :wl.r]
            flagged = int(ws[fo: fo + 4 * ns].cpu().view(torch.int32).sum().item())
        return y.cpu(), h, flagged
    args = (wl.M, wl.N, wl.K, L.dtype_code(d["x"]), L.dtype_code(d["w"]), L.dtype_code(d["b"]) if "b" in d else 0)
    nb = L.linear_workspace_size(*args)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    y = L.linear(d["x"], d["w"], d.get("b"), workspace=ws)
    torch.cuda.synchronize()
    fo, ns = L.linear_workspace_layout(*args)
    flagged = int(ws[fo: fo + 4 * ns].cpu().view(torch.int32).sum().item()) if ns > 0 else None
    return y.cpu(), None, flagged


def oracle_forward(inputs: Dict[str, torch.Tensor], wl: WL.Workload, rows=None, scale: Optional[float] = None):
    bits = {k: WL.raw_bits(v) for k, v in inputs.items()}
    dt = {k: WL.dtype_code(v) for k, v in inputs.items()}
    lora = wl.kind == "lora"
    return oracle.forward(bits["x"], dt["x"], bits["w"], dt["w"], bits.get("b"), dt.get("b"),
                          bits.get("down"), dt.get("down"), bits.get("up"), dt.get("up"),
                          scale=(wl.scale if scale is None else scale), rows=rows, lora=lora)


def score(y_gpu: torch.Tensor, res, rows, K: int, r: int):
    """Per-element tolerance check and ULP report of the GPU rows against the oracle."""
    o_dt, c_dt = res["output"], res["compute"]
    g_all = oracle.as_float64(WL.raw_bits(y_gpu), o_dt)
    g = g_all if rows is None else g_all[np.asarray(rows)]
    ref_y = oracle.as_float64(res["y"], o_dt)
    tol = oracle.tolerance(ref_y, c_dt, K, r)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - ref_y)
        same = (g == ref_y) | (np.isnan(g) & np.isnan(ref_y))
        ok = same | (err <= tol)
        # at the overflow threshold (max + half an ulp) either side is within tolerance
        fmax = {oracle.F16: 65504.0, oracle.BF16: 3.3895313892515355e38, oracle.F32: 3.4028234663852886e38}[o_dt]
        half = {oracle.F16: 16.0, oracle.BF16: 2.0 ** 119, oracle.F32: 2.0 ** 103}[o_dt]
        thr = fmax + half
        near = np.abs(np.abs(res["ref"]) - thr) <= oracle.tolerance(np.full(ref_y.shape, thr), c_dt, K, r)
        ok |= near & (np.abs(g) >= fmax) & (np.abs(ref_y) >= fmax) & (np.sign(g) == np.sign(ref_y))
    finite = np.isfinite(ref_y) & np.isfinite(g)
    worst = float(np.max(err[finite] / tol[finite])) if finite.any() else 0.0
    umax, urms = oracle.ulp_report(g[finite], res["ref"][finite], c_dt)
    bad = np.argwhere(~ok)
    return {"fail": int((~ok).sum()), "n": int(ok.size), "worst": worst, "ulp_max": umax, "ulp_rms": urms,
            "first_bad": bad[:5].tolist(), "compute": c_dt, "output": o_dt}


def sample_rows(M: int, n: int, seed: int = 0, tile: int = 256):
    """Rows to check: first/last, both sides of tile edges, and random ones."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for t in (64, 128, 192, tile):
        for b in range(t, M, t * max(1, M // (4 * t))):
            rows.update({b - 1, b})
    rows.update(rng.integers(0, M, size=n).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)
