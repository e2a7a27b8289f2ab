"""Exact-rational helpers for pinning the oracle (test side only).

Nothing here is shared with the oracle or with the GPU library.  Values are
``fractions.Fraction``; rounding is done by *searching* the neighbours of a
value among representable numbers (found with numpy/torch conversions and
``nextafter``), comparing exact distances, and breaking ties towards the even
bit pattern.  That is a different construction from the oracle's, so a slip
in either shows up as a disagreement.
"""
from __future__ import annotations

import math
import os
import re
from fractions import Fraction
from typing import Dict, List

import numpy as np
import torch

F16, BF16, F32 = 1, 2, 3
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_EMAX = {F16: 15, BF16: 127, F32: 127}
_P = {F16: 11, BF16: 8, F32: 24}

# ---- decoding stored values --------------------------------------------------


def to_fraction_array(bits: np.ndarray, dt: int) -> List[Fraction]:
    """Storage -> exact Fractions, via library conversions to float64."""
    if dt == F16:
        f = np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    elif dt == BF16:
        f = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        f = np.asarray(bits, dtype=np.float32).astype(np.float64)
    return [Fraction(float(v)) for v in f.ravel()]


# ---- neighbour-search rounding ----------------------------------------------

def _bits_of(v: float, dt: int) -> int:
    if dt == F16:
        return int(np.array([v], dtype=np.float16).view(np.uint16)[0])
    if dt == BF16:
        return int(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def _value_of(bits: int, dt: int) -> float:
    if dt == F16:
        return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])
    if dt == BF16:
        return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])
    return float(np.array([bits], dtype=np.uint32).view(np.float32)[0])


def _finite_max(dt: int) -> Fraction:
    return Fraction(2 - Fraction(2) ** (1 - _P[dt])) * Fraction(2) ** _EMAX[dt]


def exact_round(v: Fraction, dt: int):
    """Nearest value of dtype dt to the exact rational v, ties to the even bit
    pattern; +-inf past the overflow point.  Returns a Fraction or a float inf."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    mx = _finite_max(dt)
    if a > mx:
        # as if the exponent range went on: the next value would be 2^(emax+1)
        nxt = Fraction(2) ** (_EMAX[dt] + 1)
        return sign * math.inf if (a - mx) >= (nxt - a) else sign * mx
    approx = float(a)
    b0 = _bits_of(approx, dt)
    mask_max = (0x7BFF if dt == F16 else 0x7F7F if dt == BF16 else 0x7F7FFFFF)
    cands = set()
    for b in (b0 - 1, b0, b0 + 1):
        if 0 <= b <= mask_max:
            cands.add(b)
    best = None
    for b in sorted(cands):
        d = abs(Fraction(_value_of(b, dt)) - a)
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return sign * Fraction(_value_of(best[1], dt))


# ---- exact forward (tiny shapes) ----------------------------------------------

def exact_forward(x, x_dt, w, w_dt, c_dt, o_dt, b=None, b_dt=None, down=None, d_dt=None, up=None, u_dt=None,
                  scale=1, lora=True):
    """The forward in exact rational arithmetic, for a handful of outputs.
    Returns (y [M][N] as Fractions/inf, h_r [M][r])."""
    M, K = x.shape
    N = w.shape[0]
    X = np.array(to_fraction_array(x, x_dt), dtype=object).reshape(M, K)
    W = np.array(to_fraction_array(w, w_dt), dtype=object).reshape(N, K)
    Xc = np.vectorize(lambda v: exact_round(v, c_dt), otypes=[object])(X)
    Wc = np.vectorize(lambda v: exact_round(v, c_dt), otypes=[object])(W)
    B = to_fraction_array(b, b_dt) if b is not None else [Fraction(0)] * N
    sc = Fraction(scale)
    hr = None
    if lora:
        r = down.shape[0]
        D = np.array(to_fraction_array(down, d_dt), dtype=object).reshape(r, K)
        U = np.array(to_fraction_array(up, u_dt), dtype=object).reshape(N, r)
        Dc = np.vectorize(lambda v: exact_round(v, c_dt), otypes=[object])(D)
        Uc = np.vectorize(lambda v: exact_round(v, c_dt), otypes=[object])(U)
        hr = [[exact_round(sum((Xc[m, k] * Dc[j, k] for k in range(K)), Fraction(0)), c_dt) for j in range(r)]
              for m in range(M)]
    y = []
    for m in range(M):
        row = []
        for n in range(N):
            p = sum((Xc[m, k] * Wc[n, k] for k in range(K)), Fraction(0))
            if lora:
                f = sum((hr[m][j] * Uc[n, j] for j in range(down.shape[0])), Fraction(0))
                row.append(exact_round(p + sc * f + B[n], o_dt))
            else:
                pr = exact_round(p, o_dt)
                row.append(exact_round(pr + B[n], o_dt))
        y.append(row)
    return y, hr


# ---- golden fixtures ---------------------------------------------------------

_TOKEN = re.compile(r"([+-]?)(?:(\d+)\*2\^(-?\d+)|2\^(-?\d+)|(\d+(?:\.\d+)?))")


def parse_value(s: str) -> Fraction:
    """Parse an exact dyadic expression such as '-3*2^-10+2^-20' or '1'."""
    s = s.replace(" ", "")
    total, pos = Fraction(0), 0
    while pos < len(s):
        m = _TOKEN.match(s, pos)
        if not m or m.end() == pos:
            raise ValueError(f"bad value {s!r} at {pos}")
        sign = -1 if m.group(1) == "-" else 1
        if m.group(2):
            total += sign * int(m.group(2)) * Fraction(2) ** int(m.group(3))
        elif m.group(4):
            total += sign * Fraction(2) ** int(m.group(4))
        else:
            total += sign * Fraction(m.group(5))
        pos = m.end()
    return total


def load_fixtures() -> List[Dict]:
    out, cur = [], None
    with open(os.path.join(GOLDEN, "fixtures.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "name":
                cur = {"name": vals[0], "wrong": []}
                out.append(cur)
            elif key in ("kind", "dtype", "cite"):
                cur[key] = " ".join(vals)
            elif key == "wrong":
                cur["wrong"].append((parse_value(vals[0]), vals[1]))
            elif key in ("expect", "scale"):
                cur[key] = parse_value(vals[0])
            else:
                cur[key] = [parse_value(v) for v in vals]
    return out


def fixture_arrays(fx: Dict, K: int = 8):
    """Storage arrays for a fixture: x [1,K], w [1,K], b [1], down [r,K], up [1,r]."""
    dt = {"f16": F16, "bf16": BF16}[fx["dtype"]]

    def enc(vals):
        a = np.array([float(v) for v in vals], dtype=np.float64)
        assert all(Fraction(float(v)) == v for v in vals)
        if dt == F16:
            out = a.astype(np.float16)
            assert np.all(out.astype(np.float64) == a), "fixture value not representable in fp16"
            return out.view(np.uint16)
        t = torch.tensor(a, dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
        assert np.all(t.to(torch.float64).numpy() == a), "fixture value not representable in bf16"
        return t.view(torch.int16).numpy().view(np.uint16)

    def pad(vals):
        return list(vals) + [Fraction(0)] * (K - len(vals))

    arr = {"dt": dt, "x": enc(pad(fx["x"])).reshape(1, K), "w": enc(pad(fx["w"])).reshape(1, K)}
    arr["b"] = enc(fx["b"]).reshape(1) if "b" in fx else None
    if fx["kind"] == "lora":
        r = 1
        arr["down"] = enc(pad(fx["down"])).reshape(r, K)
        arr["up"] = enc(fx["up"]).reshape(1, r)
        arr["scale"] = float(fx["scale"])
    return arr


def load_policy_table():
    name = {"f16": F16, "bf16": BF16, "f32": F32}
    rows = []
    with open(os.path.join(GOLDEN, "policy_table.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            t = line.split()
            if t[2] == "REJECT":
                rows.append((name[t[0]], name[t[1]], None, None))
            else:
                rows.append((name[t[0]], name[t[1]], name[t[2]], name[t[3]]))
    return rows
