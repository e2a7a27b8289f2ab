"""The h rounding guard flags what its stated bound says it flags.

The h pass marks an element (m, j) for fp64 re-evaluation when the interval
[h - E, h + E] straddles a rounding boundary of the 16-bit compute format, with

    E = 38 * 2^-24 * (|x_m| |b_lo,j| + |x_lo,m| (|b_j| + |b_lo,j|)) + 2^-37 |x_m| |b_j| + K 2^-120

where v = v_hi + v_lo is the split of every 64-k block of a row on the grid
2^(floor(log2 max|v|) - 8).  A guard whose E came out too small (a wrong norm,
a dropped term) would still pass the element-wise parity tests as long as no
rounding happened to flip, so the number of flagged elements is checked here
against the same bound evaluated on the CPU from the exact h and exact norms.
The two may differ only where the GPU's fp32-partial h and the exact h fall on
different sides of the flagging edge, and by the GPU's slightly inflated norms:
a few percent at most.
"""
import numpy as np
import pytest
import torch

import workloads as WL
from tests.gpu_cases import gpu_forward

pytestmark = pytest.mark.gpu


def _split(v: np.ndarray):
    """hi/lo split of every 64-k block of each row (round to nearest even on the grid)."""
    rows, K = v.shape
    pad = (-K) % 64
    vb = np.pad(v, ((0, 0), (0, pad))).reshape(rows, -1, 64)
    mx = np.abs(vb).max(axis=2, keepdims=True)
    g = np.floor(np.log2(np.where(mx > 0, mx, 1.0))) - 8
    q = np.ldexp(1.0, g.astype(np.int64))
    hi = np.round(vb / q) * q
    lo = (vb - hi).reshape(rows, -1)[:, :K]
    return lo


def _expected_flags(inputs, ct, b_name="down") -> int:
    x = inputs["x"].to(ct).double().numpy()
    b = inputs[b_name].to(ct).double().numpy()
    h = x @ b.T
    xl, bl = _split(x), _split(b)
    xn = np.linalg.norm(x, axis=1)[:, None]
    xln = np.linalg.norm(xl, axis=1)[:, None]
    bn = np.linalg.norm(b, axis=1)[None, :]
    bln = np.linalg.norm(bl, axis=1)[None, :]
    E = 38 * 2.0 ** -24 * (xn * bln + xln * (bn + bln)) + 2.0 ** -37 * xn * bn + x.shape[1] * 2.0 ** -120

    def r16(v):
        return torch.from_numpy(v).to(ct).double().numpy()   # fp64 -> 16-bit, round to nearest even

    return int((r16(h - E) != r16(h + E)).sum())


# sizes that run the h pass in the work split of the full workload
@pytest.mark.parametrize("name,M,K", [("lora_f16_4096x3072x3072_r16", 4096, 3072),
                                      ("lora_bf16x_f32w_8192x4096x4096_r64", 8192, 1024),
                                      ("lora_bf16_16384x8192x8192_r128", 16384, 512)])
def test_guard_flag_count_matches_its_bound(name, M, K):
    wl = WL.WORKLOADS[name].resized(M=M, K=K)
    inputs = WL.generate(wl)
    ct = torch.float16 if torch.float16 in (inputs["x"].dtype, inputs["w"].dtype) else torch.bfloat16
    _, _, flagged = gpu_forward(inputs, wl)
    want = _expected_flags(inputs, ct)
    print(name, "M", M, "flagged", flagged, "bound says", want)
    assert want > 0
    assert abs(flagged - want) <= max(5, 0.05 * want), (flagged, want)


@pytest.mark.parametrize("M", [1024, 128])
def test_affine_guard_flag_count_matches_its_bound(M):
    """The plain affine form guards the rounding of p = x.W^T to the fp16 output
    with the same bound (b = W); M = 128 runs the narrow-column split."""
    wl = WL.WORKLOADS["affine_f16_1024x768x1024"].resized(M=M)
    inputs = WL.generate(wl)
    _, _, flagged = gpu_forward(inputs, wl)
    want = _expected_flags(inputs, torch.float16, b_name="w")
    print(wl.name, "flagged", flagged, "bound says", want)
    assert want > 0
    assert abs(flagged - want) <= max(5, 0.05 * want), (flagged, want)
