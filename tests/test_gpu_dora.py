"""GPU parity of DoRA: the row norms of the merged weight and the DoRA forward,
through the C ABI, against the fp64 oracle.

Bar: norms within 2^-24 (16 + K/64) relative (fp32 sums of squares: E
elements per lane, a 16/32-lane butterfly, K/128 tile partials added in order,
and the fp32 merged value itself); y within the forward's per-element
tolerance of its compute dtype, the GPU using its own norms and the oracle its
own.
"""
import numpy as np
import pytest
import torch

import lora_bypass_linear_amd as L
import oracle
import workloads as WL
from tests.gpu_cases import say, sample_rows, score

pytestmark = pytest.mark.gpu

BASE = WL.WORKLOADS


def _norm_check(wl, rows=None, scale=None):
    inp = WL.generate(wl.resized(M=1))
    w, d, u = inp["w"], inp["down"], inp["up"]
    s = wl.scale if scale is None else scale
    say("dora norms", wl.name, f"N={wl.N} K={wl.K} r={wl.r}")
    g = L.dora_norms(w.cuda(), d.cuda(), u.cuda(), s)
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    want, exact, _ = oracle.dora_norms(WL.raw_bits(w), WL.dtype_code(w), WL.raw_bits(d), WL.dtype_code(d),
                                       WL.raw_bits(u), WL.dtype_code(u), scale=s, rows=rows)
    got = g if rows is None else g[np.asarray(rows)]
    rel = np.abs(got - exact) / np.maximum(exact, 1e-30)
    bound = 2.0 ** -24 * (16 + wl.K / 64)
    print(wl.name, "norms n", got.size, "max rel err", float(rel.max()), "bound", bound)
    assert np.all(rel <= bound), (float(rel.max()), bound)


def _fwd_check(wl, rows=None):
    inp = WL.generate(wl)
    mag = WL.generate_magnitude(wl)
    d = {k: v.cuda() for k, v in inp.items()}
    say("dora forward", wl.name, f"M={wl.M} N={wl.N} K={wl.K} r={wl.r}")
    norms = L.dora_norms(d["w"], d["down"], d["up"], wl.scale)
    y = L.dora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, mag.cuda(), norms, d.get("b"))
    torch.cuda.synchronize()
    b = {k: WL.raw_bits(v) for k, v in inp.items()}
    dt = {k: WL.dtype_code(v) for k, v in inp.items()}
    res = oracle.dora_forward(b["x"], dt["x"], b["w"], dt["w"], b.get("b"), dt.get("b"), b["down"], dt["down"],
                              b["up"], dt["up"], WL.raw_bits(mag), WL.dtype_code(mag), scale=wl.scale, rows=rows)
    s = score(y.cpu(), res, rows, wl.K, wl.r)
    print(wl.name, {k: v for k, v in s.items() if k != "first_bad"})
    assert s["fail"] == 0, s


SMALL = {
    "lora_f16_4096x3072x3072_r16": dict(M=300, K=392, N=336),
    "lora_bf16x_f32w_8192x4096x4096_r64": dict(M=257, K=264, N=200),
    "lora_bf16_16384x8192x8192_r128": dict(M=270, K=520, N=304),
    "sweep_xf32_wf32_2048x1280x5120_r32": dict(M=100, K=72, N=136),
    "sweep_xbf16_wf16_2048x1280x5120_r32": None,
}
SMALL = {k: v for k, v in SMALL.items() if v}


@pytest.mark.parametrize("name", list(SMALL))
def test_norms_small(name):
    _norm_check(BASE[name].resized(**SMALL[name]))


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    _fwd_check(BASE[name].resized(**SMALL[name]))


@pytest.mark.parametrize("K", [76, 2, 130])   # rows not a multiple of the lane chunk: the element path
def test_norms_ragged_k(K):
    _norm_check(BASE["lora_f16_4096x3072x3072_r16"].resized(N=70, K=K))


@pytest.mark.parametrize("name", ["lora_bf16_16384x8192x8192_r128", "lora_f16_4096x3072x3072_r16"])
def test_norms_many_tiles_ragged(name):
    """2145 tiles of 128 x 128, ragged in N and K, more than the resident
    workgroups (several rounds per CU)."""
    _norm_check(BASE[name].resized(N=8197, K=4104))


def test_norms_rank_zero_and_negative_scale():
    _norm_check(BASE["lora_bf16_16384x8192x8192_r128"].resized(N=130, K=136, r=0))
    _norm_check(BASE["lora_bf16_16384x8192x8192_r128"].resized(N=130, K=136, r=17), scale=-0.5)


@pytest.mark.parametrize("name", ["lora_f16_4096x3072x3072_r16", "lora_bf16x_f32w_8192x4096x4096_r64",
                                  "lora_bf16_16384x8192x8192_r128"])
def test_norms_full_size_sampled(name):
    wl = BASE[name]
    _norm_check(wl, rows=sample_rows(wl.N, 48, seed=wl.seed, tile=128))


def test_forward_full_size_sampled():
    wl = BASE["lora_f16_4096x3072x3072_r16"]
    _fwd_check(wl, rows=sample_rows(wl.M, 24, seed=wl.seed))
