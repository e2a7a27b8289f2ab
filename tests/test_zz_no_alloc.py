"""The allocation-free forward (lyc_lora_linear_fwd_noalloc) against the
workspace forward (lyc_lora_linear_fwd), both called through the C ABI on the
same seeded inputs: bitwise-identical outputs, and both within the oracle's
per-element tolerance.  Calls in a row share the library's static scratch
array, so each later call (smaller input, other dtypes, a K split) must not
see what the one before left there."""
import ctypes

import pytest
import torch

import lora_bypass_linear_amd as L
import workloads as WL
from tests.gpu_cases import oracle_forward, sample_rows, say, score

pytestmark = pytest.mark.gpu

# largest first, then smaller inputs: the fp16 rank-16 shape at decode-sized M
# (its GEMM splits K: fp32 partial sums in the scratch array), fp32 master
# weights (bf16 copies of W, down and up in the scratch array)
CASES = [
    ("lora_bf16_16384x8192x8192_r128", dict(M=1000, N=520, K=1032)),
    ("lora_f16_4096x3072x3072_r16", dict(M=16, N=1024, K=3072)),
    ("lora_bf16x_f32w_8192x4096x4096_r64", dict(M=200, N=264, K=512)),
    ("lora_f16_4096x3072x3072_r16", dict(M=130, N=136, K=264)),
]


def _call_noalloc(d, wl, y):
    b = d.get("b")
    st = L.lib().lyc_lora_linear_fwd_noalloc(
        ctypes.c_void_p(d["x"].data_ptr()), L.dtype_code(d["x"]), ctypes.c_void_p(d["w"].data_ptr()),
        L.dtype_code(d["w"]), None if b is None else ctypes.c_void_p(b.data_ptr()), 0 if b is None else L.dtype_code(b),
        ctypes.c_void_p(d["down"].data_ptr()), L.dtype_code(d["down"]), ctypes.c_void_p(d["up"].data_ptr()),
        L.dtype_code(d["up"]), wl.r, ctypes.c_double(wl.scale), ctypes.c_void_p(y.data_ptr()), L.dtype_code(y),
        wl.M, wl.N, wl.K, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == L.OK, L.lib().lyc_status_str(st)


def test_noalloc_matches_workspace_forward():
    dev = torch.device("cuda:0")
    for name, dims in CASES:
        wl = WL.WORKLOADS[name].resized(**dims)
        inputs = WL.generate(wl)
        d = {k: v.to(dev) for k, v in inputs.items()}
        say("noalloc", wl.name, dims)
        y_ref = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"))
        y = torch.full_like(y_ref, float("nan"))
        _call_noalloc(d, wl, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if y.element_size() == 2 else y.view(torch.int32),
                           y_ref.view(torch.int16) if y.element_size() == 2 else y_ref.view(torch.int32)), wl.name
        rows = sample_rows(wl.M, 48, seed=wl.seed)
        s = score(y.cpu(), oracle_forward(inputs, wl, rows=rows), rows, wl.K, wl.r)
        assert s["fail"] == 0, (wl.name, s)


def test_noalloc_binding_and_refusal():
    dev = torch.device("cuda:0")
    wl = WL.WORKLOADS["lora_f16_4096x3072x3072_r16"].resized(M=64, N=128, K=256)
    d = {k: v.to(dev) for k, v in WL.generate(wl).items()}
    say("noalloc binding", wl.name)
    y = L.lora_linear_noalloc(d["x"], d["w"], d["down"], d["up"], wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(y, L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale))
    # a problem whose scratch need exceeds the array is refused before any launch
    big = WL.WORKLOADS["lora_bf16x_f32w_8192x4096x4096_r64"].resized(M=16, N=16384, K=4096)
    assert L.lora_workspace_size(big.M, big.N, big.K, big.r, 2, 3, 0, 3, 3) > L.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((big.M, big.K), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((big.N, big.K), dtype=torch.float32, device=dev)
    dn = torch.zeros((big.r, big.K), dtype=torch.float32, device=dev)
    up = torch.zeros((big.N, big.r), dtype=torch.float32, device=dev)
    with pytest.raises(L.LycError) as e:
        L.lora_linear_noalloc(x, w, dn, up, 1.0)
    assert e.value.status == L.ERR_SCRATCH
