"""What the exact-rounding contraction assumes about gfx950 MFMA steps,
checked on the GPU against exact host arithmetic (test-side probe kernel in
tests/probe/):

  * the lane layouts of A, B and the 16x16 result that the kernels use;
  * a 16-bit step whose products and partial sums are integers below 2^23 on
    one common grid is exact, also when chained on such a result (the hi x hi
    part of the split contraction);
  * one step that adds products of absolute sum S to an accumulator C errs by
    less than B * 2^-24 * (|C| + S), B = half the library's cross-chain factor;
  * fp16 subnormal inputs are not flushed.
The printed figures are the measurements the constants were chosen from.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from tests.gpu_cases import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE = os.path.join(HERE, "probe", "libmfma_probe.so")
SRC = os.path.join(os.path.dirname(HERE), "lora_bypass_linear_amd", "csrc", "hpass.hip")


def step_factor():
    return float(re.search(r"STEP_ERR\s*=\s*([0-9.]+)", open(SRC).read()).group(1))


def check_model(A, B, D, C=None):
    """err <= B * 2^-24 (|C| + S) elementwise; returns the largest fraction of the bound used."""
    C = np.zeros(D.shape) if C is None else C
    E = exact(A, B, C)
    S = np.einsum("tik,tjk->tij", np.abs(A), np.abs(B)) + np.abs(C)
    bound = step_factor() * 2.0 ** -24 * S
    err = np.abs(D - E)
    assert np.all(err <= bound), float(np.max(err / np.where(bound > 0, bound, 1)))
    return float(np.max(np.where(bound > 0, err / bound, 0.0)))


def _lib():
    L = ctypes.CDLL(PROBE)
    L.probe_mfma16.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    return L


def _bits(vals, dt):
    t = torch.from_numpy(np.asarray(vals, dtype=np.float32))
    t = t.to(torch.float16 if dt == 1 else torch.bfloat16)
    return t


def run(dt, a, bt, c):
    """a: [T,16,32], bt: [T,16,32] (float values representable in dt), c: [T,16,16] fp32."""
    dev = torch.device("cuda:0")
    A = _bits(a, dt).to(dev).contiguous()
    B = _bits(bt, dt).to(dev).contiguous()
    C = torch.from_numpy(np.asarray(c, np.float32)).to(dev).contiguous()
    D = torch.empty_like(C)
    T = a.shape[0]
    say("mfma probe", dt, T)
    st = _lib().probe_mfma16(dt, A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), T,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    return (A.cpu().double().numpy(), B.cpu().double().numpy(), D.cpu().double().numpy())


def exact(a, bt, c):
    # products of 16-bit values are exact in fp64; these sums stay within 53 bits
    return np.einsum("tik,tjk->tij", a, bt) + c


@pytest.mark.parametrize("dt", [1, 2])
def test_lane_layout_exact(dt):
    rng = np.random.default_rng(0)
    T = 64
    a = rng.integers(-4, 5, size=(T, 16, 32)).astype(np.float64)
    bt = rng.integers(-4, 5, size=(T, 16, 32)).astype(np.float64)
    c = rng.integers(-64, 65, size=(T, 16, 16)).astype(np.float64)
    A, B, D = run(dt, a, bt, c)
    np.testing.assert_array_equal(D, exact(A, B, c))


def _ratio(dt, a, bt):
    A, B, D = run(dt, a, bt, np.zeros((a.shape[0], 16, 16)))
    E = exact(A, B, 0.0)
    S = np.einsum("tik,tjk->tij", np.abs(A), np.abs(B))
    err = np.abs(D - E)
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(S > 0, err / (2.0 ** -24 * S), 0.0)
    rne = np.mean(D == E.astype(np.float32).astype(np.float64))
    used = check_model(A, B, D)
    print(f"  fraction of the step bound used: {used:.4f}")
    return float(ratio.max()), float(rne)


@pytest.mark.parametrize("dt", [1, 2])
def test_step_error_gaussian(dt):
    rng = np.random.default_rng(1)
    T = 4096
    mx, rne = _ratio(dt, rng.standard_normal((T, 16, 32)), rng.standard_normal((T, 16, 32)) / 40)
    print(f"dt={dt} gaussian: max err / (2^-24 sum|ab|) = {mx:.4f}; results equal to RNE32(exact): {rne:.5f}")


@pytest.mark.parametrize("dt", [1, 2])
def test_step_error_wide_exponents(dt):
    """Magnitudes spread over 2^-12 .. 2^12 with random signs: heavy alignment
    shifts and cancellation inside one step."""
    rng = np.random.default_rng(2)
    T = 4096
    a = rng.choice([-1, 1], size=(T, 16, 32)) * 2.0 ** rng.integers(-12, 12, size=(T, 16, 32)) * \
        (1 + rng.integers(0, 128, size=(T, 16, 32)) / 128)
    bt = rng.choice([-1, 1], size=(T, 16, 32)) * 2.0 ** rng.integers(-12, 12, size=(T, 16, 32)) * \
        (1 + rng.integers(0, 128, size=(T, 16, 32)) / 128)
    mx, rne = _ratio(dt, a, bt)
    print(f"dt={dt} wide: max err / (2^-24 sum|ab|) = {mx:.4f}; results equal to RNE32(exact): {rne:.5f}")


def test_fp16_subnormals_kept():
    T = 16
    a = np.zeros((T, 16, 32))
    bt = np.zeros((T, 16, 32))
    a[:, :, 0] = 1.0
    a[:, :, 1] = 2.0 ** -20          # fp16 subnormal
    a[:, :, 2] = 2.0 ** -24          # smallest fp16 subnormal
    bt[:, :, 0] = 2.0 ** -3
    bt[:, :, 1] = 1.0
    bt[:, :, 2] = 1.0
    A, B, D = run(1, a, bt, np.zeros((T, 16, 16)))
    np.testing.assert_array_equal(D, exact(A, B, 0.0))


@pytest.mark.parametrize("dt", [1, 2])
def test_step_error_dominant_term(dt):
    """One dominant product and 31 small ones placed 2^-20 .. 2^-31 below it:
    probes how many bits below the leading product one step keeps."""
    rng = np.random.default_rng(3)
    T = 16 * 12
    a = np.zeros((T, 16, 32))
    bt = np.zeros((T, 16, 32))
    a[:, :, 0] = 16.0
    bt[:, :, 0] = 16.0                                   # leading product 2^8
    shift = np.repeat(np.arange(-4, 8), 16)              # small products at 2^(8-24-shift)
    for t in range(T):
        s = shift[t]
        a[t, :, 1:] = 2.0 ** -7
        frac = 1 + rng.integers(0, 8, size=(16, 31)) / 8
        sign = rng.choice([-1.0, 1.0], size=(16, 31)) if t % 2 else 1.0
        bt[t, :, 1:] = sign * 2.0 ** -(9 + s) * frac
    A, B, D = run(dt, a, bt, np.zeros((T, 16, 16)))
    E = exact(A, B, 0.0)
    S = np.einsum("tik,tjk->tij", np.abs(A), np.abs(B))
    ratio = np.abs(D - E) / (2.0 ** -24 * S)
    for s in range(-4, 8):
        sel = shift == s
        print(f"dt={dt} small terms at 2^-{24 + s} of the leading one: max ratio {ratio[sel].max():.3f}")
    print(f"  fraction of the step bound used: {check_model(A, B, D):.4f}")


@pytest.mark.parametrize("dt", [1, 2])
def test_step_alignment_reference(dt):
    """16 equal leading products (their sum is 16x the largest product) and 16
    small ones 2^-20 .. 2^-27 below a leading product.  If a step aligned the
    small terms to the running sum rather than to the largest product, they
    would lose up to 4 more bits; the printed ratios tell which."""
    rng = np.random.default_rng(4)
    T = 16 * 8
    a = np.zeros((T, 16, 32))
    bt = np.zeros((T, 16, 32))
    a[:, :, :16] = 16.0
    bt[:, :, :16] = 16.0                                 # 16 products of 2^8, sum 2^12
    shift = np.repeat(np.arange(-4, 4), 16)
    for t in range(T):
        a[t, :, 16:] = 2.0 ** -7
        bt[t, :, 16:] = 2.0 ** -(9 + shift[t]) * (1 + rng.integers(0, 8, size=(16, 16)) / 8)
    A, B, D = run(dt, a, bt, np.zeros((T, 16, 16)))
    E = exact(A, B, 0.0)
    err = np.abs(D - E)
    for s in range(-4, 4):
        sel = shift == s
        print(f"dt={dt} 16 leading terms, small terms at 2^-{24 + s} of one: max err in units of "
              f"2^-24*(largest product) {np.max(err[sel] / (2.0 ** -24 * 256.0)):.3f}")
    print(f"  fraction of the step bound used: {check_model(A, B, D):.4f}")


def test_fp32_step_layout_exact():
    """The fp32 step the kernels use (four chained 16x16x4 f32 MFMAs over one
    16-byte fragment per lane) computes a 16x16x16 product exactly on small
    integers."""
    L = ctypes.CDLL(PROBE)
    L.probe_mfma32.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    rng = np.random.default_rng(6)
    T = 32
    a = rng.integers(-4, 5, size=(T, 16, 16)).astype(np.float32)
    bt = rng.integers(-4, 5, size=(T, 16, 16)).astype(np.float32)
    c = rng.integers(-64, 65, size=(T, 16, 16)).astype(np.float32)
    dev = torch.device("cuda:0")
    A, B, C = (torch.from_numpy(v).to(dev) for v in (a, bt, c))
    D = torch.empty_like(C)
    say("mfma fp32 probe", T)
    assert L.probe_mfma32(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), T,
                          torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = D.cpu().numpy().astype(np.float64)
    want = np.einsum("tik,tjk->tij", a.astype(np.float64), bt.astype(np.float64)) + c
    if not np.array_equal(got, want):
        # report which k pairing the hardware used, to fix the fragment layout
        print("fp32 step mismatch; first block got\n", got[0, :4, :4], "\nwant\n", want[0, :4, :4])
    np.testing.assert_array_equal(got, want)


def _split(v, dt):
    """hi/lo split of [T,16,64] blocks as the kernels do it: hi = v rounded to
    the grid 2^(floor(log2 max|v|) - 8) of its row's 64-k block, lo = v - hi."""
    mx = np.abs(v).max(axis=-1, keepdims=True)
    e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
    q = 2.0 ** (e - 8)
    hi = np.rint(v / q) * q
    return hi, v - hi


@pytest.mark.parametrize("dt", [1, 2])
@pytest.mark.parametrize("kind", ["gaussian", "lognormal", "wide", "extreme"])
def test_split_hi_steps_exact(dt, kind):
    """Two chained 32-k steps of hi parts (one 64-k block) are exact.
    "extreme": one sign per row, most elements just below 2 (hi parts of 2^9
    grid units under fp16, 510 under bf16) and a quarter of them small grid
    multiples (1..255 units), so that the block's sum comes within 2^18 units
    of the 2^24 the exactness argument allows and needs every low bit."""
    rng = np.random.default_rng(7)
    T = 512
    if kind == "gaussian":
        x, d = rng.standard_normal((T, 16, 64)), rng.standard_normal((T, 16, 64)) / 64
    elif kind == "lognormal":
        x = rng.standard_normal((T, 16, 64)) * np.exp(rng.standard_normal((T, 16, 1)) * 2)
        d = rng.standard_normal((T, 16, 64)) * np.exp(rng.standard_normal((T, 16, 1)))
    elif kind == "wide":
        x = rng.choice([-1, 1], (T, 16, 64)) * 2.0 ** rng.integers(-10, 10, (T, 16, 64))
        d = rng.choice([-1, 1], (T, 16, 64)) * 2.0 ** rng.integers(-10, 10, (T, 16, 64))
    else:
        top = 2.0 - (2.0 ** -10 if dt == 1 else 2.0 ** -7)
        small = lambda: rng.integers(1, 256, (T, 16, 64)) * 2.0 ** -8
        pick = lambda: rng.random((T, 16, 64)) < 0.25
        x = np.where(pick(), small(), top) * rng.choice([-1, 1], (T, 1, 1))
        d = np.where(pick(), small(), top) * rng.choice([-1, 1], (T, 1, 1))
        x[:, :, 0] = d[:, :, 0] = top                       # every row keeps its block maximum
    x = _bits(x, dt).double().numpy()
    d = _bits(d, dt).double().numpy()
    xh, _ = _split(x, dt)
    dh, _ = _split(d, dt)
    assert np.array_equal(_bits(xh, dt).double().numpy(), xh)   # representable
    A1, B1, D1 = run(dt, dh[:, :, :32], xh[:, :, :32], np.zeros((T, 16, 16)))
    A2, B2, D2 = run(dt, dh[:, :, 32:], xh[:, :, 32:], D1)
    want = np.einsum("tik,tjk->tij", dh, xh)
    np.testing.assert_array_equal(D2, want)


@pytest.mark.parametrize("dt", [1, 2])
def test_step_error_with_accumulator(dt):
    """Cross-chain shape: a large accumulator plus small products, and the
    reverse, against the step bound."""
    rng = np.random.default_rng(8)
    T = 2048
    a = rng.standard_normal((T, 16, 32))
    b = rng.standard_normal((T, 16, 32)) * 2.0 ** rng.integers(-12, 2, (T, 16, 1))
    c = rng.standard_normal((T, 16, 16)) * 2.0 ** rng.integers(-6, 8, (T, 1, 1))
    c = c.astype(np.float32).astype(np.float64)
    A, B, D = run(dt, a, b, c)
    used = check_model(A, B, D, c)
    print(f"dt={dt} step with accumulator: fraction of the step bound used: {used:.4f}")
