"""What the h guard assumes about one gfx950 MFMA step, checked on the GPU
against exact host arithmetic (test-side probe kernel in tests/probe/):

  * the lane layouts of A, B and the 16x16 result that the kernels use;
  * the error of one v_mfma_f32_16x16x32_{f16,bf16} step started from zero is
    at most GUARD * 2^-24 * sum_k |a_k b_k| (GUARD is the factor the library
    passes to its h guard);
  * fp16 subnormal inputs are not flushed.
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
API = os.path.join(os.path.dirname(HERE), "lora_bypass_linear_amd", "csrc", "api.cpp")


def guard_factor():
    m = re.search(r"GUARD_FACTOR\s*=\s*([0-9.]+)", open(API).read())
    return float(m.group(1))


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
    return float(ratio.max()), float(rne)


@pytest.mark.parametrize("dt", [1, 2])
def test_step_error_gaussian(dt):
    rng = np.random.default_rng(1)
    T = 4096
    mx, rne = _ratio(dt, rng.standard_normal((T, 16, 32)), rng.standard_normal((T, 16, 32)) / 40)
    print(f"dt={dt} gaussian: max err / (2^-24 sum|ab|) = {mx:.4f}; results equal to RNE32(exact): {rne:.5f}")
    assert mx <= guard_factor()


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
    assert mx <= guard_factor()


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
