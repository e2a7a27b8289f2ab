"""GPU parity of the LoRA merge W' = round_out(W + scale * up_c . down_c)
against the fp64 oracle, through the C ABI, element by element.

Bar: the per-element tolerance of the forward (fp16 2e-4 + 2e-3|ref|, bf16
2e-3 + 1.6e-2|ref|, fp32 output from 16-bit compute: the 16-bit bound; fp32
compute: 8 * 2^-24 * sqrt(r) * (1 + |ref|)); W' is checked in full at sizes
spanning several 128 x 128 tiles with ragged edges, and on sampled rows at the
full weight shapes of the benchmark workloads.
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
_T = {L.F16: torch.float16, L.BF16: torch.bfloat16, L.F32: torch.float32}


def _weights(name, N, K, r, w_dt=None, f_dt=None):
    """W [N,K], down [r,K], up [N,r] of a workload (its seeded generator), with
    W and/or the factors optionally cast to another dtype."""
    inp = WL.generate(BASE[name].resized(M=1, N=N, K=K, r=r))
    w, d, u = inp["w"], inp["down"], inp["up"]
    if w_dt is not None:
        w = w.float().to(_T[w_dt])
    if f_dt is not None:
        d, u = d.float().to(_T[f_dt]), u.float().to(_T[f_dt])
    return w, d, u


def _oracle(w, d, u, scale, rows=None):
    return oracle.merge(WL.raw_bits(w), WL.dtype_code(w), WL.raw_bits(d), WL.dtype_code(d), WL.raw_bits(u),
                        WL.dtype_code(u), scale=scale, rows=rows)


def _gpu(w, d, u, scale, tag, out=None, inplace=False):
    dev = torch.device("cuda:0")
    wg, dg, ug = w.to(dev), d.to(dev), u.to(dev)
    say("merge", tag, f"N={w.shape[0]} K={w.shape[1]} r={d.shape[0]} dts={WL.dtype_code(w)},"
        f"{WL.dtype_code(d)},{WL.dtype_code(u)} scale={scale} inplace={inplace}")
    o = L.lora_merge(wg, dg, ug, scale, out=wg if inplace else out)
    torch.cuda.synchronize()
    return o.cpu()


def _check(w, d, u, scale, tag, rows=None, **kw):
    y = _gpu(w, d, u, scale, tag, **kw)
    res = _oracle(w, d, u, scale, rows=rows)
    s = score(y, res, rows, d.shape[0], 0)
    print(tag, {k: v for k, v in s.items() if k != "first_bad"})
    assert s["fail"] == 0, s
    return y, s


# ---- the benchmark workloads' weights at oracle-friendly sizes ----------------------

SMALL = [
    ("f16_r16", "lora_f16_4096x3072x3072_r16", 333, 392, 16, None, None),
    ("f32_r64", "lora_bf16x_f32w_8192x4096x4096_r64", 200, 264, 64, None, None),
    ("bf16_r128", "lora_bf16_16384x8192x8192_r128", 300, 520, 128, None, None),
    # W and the factors in different dtypes: the policy over (W, down, up)
    ("f32w_bf16f", "lora_bf16x_f32w_8192x4096x4096_r64", 260, 136, 64, L.F32, L.BF16),
    ("f32w_f16f", "lora_bf16x_f32w_8192x4096x4096_r64", 260, 136, 64, L.F32, L.F16),
    ("bf16w_f32f", "lora_bf16_16384x8192x8192_r128", 270, 200, 128, L.BF16, L.F32),
    ("f16w_f32f", "lora_f16_4096x3072x3072_r16", 140, 300, 16, L.F16, L.F32),
]


@pytest.mark.parametrize("tag,name,N,K,r,w_dt,f_dt", SMALL, ids=[c[0] for c in SMALL])
def test_small_full_output(tag, name, N, K, r, w_dt, f_dt):
    w, d, u = _weights(name, N, K, r, w_dt, f_dt)
    _check(w, d, u, BASE[name].scale, tag)


def test_mixed_halves_refused():
    w, d, u = _weights("lora_f16_4096x3072x3072_r16", 64, 64, 8, L.F16, L.BF16)
    with pytest.raises(L.MixedHalfError):
        _gpu(w, d, u, 1.0, "mixed")


# ---- ranks, ragged and degenerate shapes, scales -------------------------------------

EDGE = [
    ("rank0_f16", 70, 72, 0, 1.0),
    ("rank1", 65, 70, 1, 1.0),
    ("rank17", 129, 136, 17, 1.0),
    ("rank33", 100, 128, 33, 0.5),
    ("rank200", 90, 264, 200, 1.0),
    ("rank256", 64, 128, 256, 1.0),
    ("one_by_one", 1, 1, 4, 1.0),
    ("k_odd", 131, 77, 16, 1.0),         # rows not 16-byte multiples: the scalar path
    ("k_two", 257, 2, 5, 1.0),
    ("n_one", 1, 1000, 16, 1.0),
    ("scale_neg", 96, 256, 32, -0.75),
    ("scale_zero", 64, 64, 16, 0.0),
    ("scale_big", 64, 64, 16, 1000.0),
]


@pytest.mark.parametrize("tag,N,K,r,scale", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("dt", [L.F16, L.BF16, L.F32])
def test_edge_cases(tag, N, K, r, scale, dt):
    w, d, u = _weights("lora_f16_4096x3072x3072_r16", N, K, r, dt, dt)
    _check(w, d, u, scale, f"{tag}_{dt}")


@pytest.mark.parametrize("tag,name,r", [("bf16", "lora_bf16_16384x8192x8192_r128", 128),
                                        ("f16_bf16out", "lora_f16_4096x3072x3072_r16", 16)])
def test_many_tiles_ragged_full_output(tag, name, r):
    """2145 tiles of 128 x 128, ragged in N and K, more than the resident
    workgroups (several rounds per CU); in place too."""
    w, d, u = _weights(name, 8197, 4104, r)
    y, _ = _check(w, d, u, BASE[name].scale, f"many tiles {tag}")
    assert torch.equal(_gpu(w, d, u, BASE[name].scale, f"many tiles {tag} in place", inplace=True), y)


def test_unaligned_factors_same_result():
    """down and up one element into their buffers: the merge prepares copies
    instead of reading them as stored, with the same W'."""
    w, d, u = _weights("lora_bf16_16384x8192x8192_r128", 300, 520, 128)
    y, _ = _check(w, d, u, 2.0, "aligned factors")
    dev = torch.device("cuda:0")

    def shift(t):   # t copied one element into a fresh buffer
        buf = torch.zeros(t.numel() + 1, dtype=t.dtype, device=dev)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    say("merge", "unaligned factors")
    y_un = L.lora_merge(w.to(dev), shift(d.to(dev)), shift(u.to(dev)), 2.0)
    torch.cuda.synchronize()
    assert torch.equal(y_un.cpu(), y)


def test_rank_zero_is_a_copy():
    w, d, u = _weights("lora_bf16_16384x8192x8192_r128", 70, 200, 0)
    y = _gpu(w, d, u, 2.0, "rank0 copy")
    assert torch.equal(y, w)


def test_fp32_weight_rounded_once_with_rank_zero():
    """fp32 W with fp16 factors: the output is fp32 (policy), W' = W exactly."""
    w, d, u = _weights("lora_bf16x_f32w_8192x4096x4096_r64", 64, 64, 0, L.F32, L.F16)
    y = _gpu(w, d, u, 1.0, "rank0 fp32")
    assert y.dtype == torch.float32 and torch.equal(y, w)


def test_in_place_matches_out_of_place():
    w, d, u = _weights("lora_bf16_16384x8192x8192_r128", 300, 520, 128)
    y_out = _gpu(w, d, u, 2.0, "out of place")
    y_in = _gpu(w, d, u, 2.0, "in place", inplace=True)
    assert torch.equal(y_in, y_out)


def test_unaligned_output():
    """W' a view one element into a buffer: element alignment only (scalar path)."""
    w, d, u = _weights("lora_f16_4096x3072x3072_r16", 130, 136, 16)
    dev = torch.device("cuda:0")
    buf = torch.zeros(130 * 136 + 1, dtype=torch.float16, device=dev)
    out = buf[1:].view(130, 136)
    y = _gpu(w, d, u, 1.0, "unaligned out", out=out)
    ref = _gpu(w, d, u, 1.0, "aligned out")
    assert torch.equal(y, ref) and buf[0].item() == 0


def test_overflow_to_inf_matches():
    w, d, u = _weights("lora_f16_4096x3072x3072_r16", 64, 64, 16)
    w = (w.float() * 3.0e6).clamp(-65504, 65504).half()
    res = _oracle(w, d, u, 4000.0)
    assert np.isinf(oracle.as_float64(res["y"], oracle.F16)).any()
    _check(w, d, u, 4000.0, "overflow")


def test_deterministic():
    w, d, u = _weights("lora_bf16_16384x8192x8192_r128", 300, 520, 128)
    assert torch.equal(_gpu(w, d, u, 2.0, "det 1"), _gpu(w, d, u, 2.0, "det 2"))


# ---- the full weight shapes of the benchmark workloads, sampled rows -----------------

FULL = ["lora_f16_4096x3072x3072_r16", "lora_bf16x_f32w_8192x4096x4096_r64", "lora_bf16_16384x8192x8192_r128"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    wl = BASE[name]
    w, d, u = _weights(name, wl.N, wl.K, wl.r)
    rows = sample_rows(wl.N, 32, seed=wl.seed, tile=128)
    _check(w, d, u, wl.scale, name, rows=rows)
