"""Python binding of liblyc.so, the gfx950 fused LoRA-bypass linear.

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  The
library must have been built (``python -m lora_bypass_linear_amd.build``);
nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = ["F16", "BF16", "F32", "LycError", "MixedHalfError", "lib", "resolve_dtypes", "linear", "lora_linear",
           "lora_linear_noalloc", "lora_merge", "lora_linear_backward", "dora_norms", "dora_linear", "linear_workspace_size", "lora_workspace_size", "lora_workspace_layout",
           "linear_workspace_layout", "linear_prepare", "lora_merge_workspace_size", "lora_bwd_workspace_size",
           "lora_bwd_workspace_layout", "gemm_tile", "gemm_plan", "lora_linear_tune", "tuning_save",
           "tuning_load", "tuning_clear", "tuning_count", "tuning_key", "tuning_lookup", "tuning_cache_path", "profile_begin", "profile_end",
           "dtype_code", "torch_dtype"]

F16, BF16, F32 = 1, 2, 3
OK, ERR_MIXED_HALF, ERR_INVALID_ARG, ERR_DTYPE_MISMATCH, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE, ERR_IO, ERR_SCRATCH = range(9)
# the static device array of lyc_lora_linear_fwd_noalloc (LYC_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
# LYC_LIB: another build of the same library (the sanitizer build of the host
# code, for the CPU test suite)
LIB_PATH = os.environ.get("LYC_LIB") or os.path.join(_HERE, "liblyc.so")
_lib = None

_CODE = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
_TORCH = {v: k for k, v in _CODE.items()}


class LycError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"lyc status {status}: {message}")
        self.status = status


class MixedHalfError(LycError, ValueError):
    pass


def lib():
    """Load liblyc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m lora_bypass_linear_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        c_i64, c_int, c_vp, c_sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.lyc_resolve_dtypes.argtypes = [ctypes.POINTER(c_int), c_int, ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
        L.lyc_linear_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_int, c_int, c_int, ctypes.POINTER(c_sz)]
        L.lyc_linear_fwd.argtypes = [c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_i64, c_i64, c_i64,
                                     c_vp, c_sz, c_vp]
        L.lyc_linear_fwd_prepared.argtypes = [c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_i64, c_i64,
                                              c_i64, c_vp, c_sz, c_vp]
        L.lyc_linear_prepare.argtypes = [c_vp, c_int, c_int, c_int, c_i64, c_i64, c_i64, c_vp, c_sz, c_vp]
        L.lyc_lora_linear_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, c_int,
                                                     ctypes.POINTER(c_sz)]
        L.lyc_lora_linear_fwd.argtypes = [c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_i64,
                                          ctypes.c_double, c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_sz, c_vp]
        L.lyc_lora_linear_fwd_noalloc.argtypes = [c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int,
                                                  c_i64, ctypes.c_double, c_vp, c_int, c_i64, c_i64, c_i64, c_vp]
        L.lyc_lora_workspace_layout.argtypes = [c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, c_int,
                                                ctypes.POINTER(c_sz), ctypes.POINTER(c_i64), ctypes.POINTER(c_sz),
                                                ctypes.POINTER(c_i64)]
        L.lyc_linear_workspace_layout.argtypes = [c_i64, c_i64, c_i64, c_int, c_int, c_int, ctypes.POINTER(c_sz),
                                                  ctypes.POINTER(c_i64)]
        L.lyc_lora_merge_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_int, c_int, c_int, ctypes.POINTER(c_sz)]
        L.lyc_lora_merge_fwd.argtypes = [c_vp, c_int, c_vp, c_int, c_vp, c_int, c_i64, ctypes.c_double, c_vp, c_int,
                                         c_i64, c_i64, c_vp, c_sz, c_vp]
        L.lyc_lora_linear_bwd_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int,
                                                         c_int, c_int, c_int, ctypes.POINTER(c_sz)]
        L.lyc_lora_linear_bwd.argtypes = [c_vp, c_int, c_vp, c_int, c_int, c_vp, c_int, c_vp, c_int, c_i64,
                                          ctypes.c_double, c_vp, c_int, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                          c_vp, c_sz, c_vp]
        L.lyc_lora_linear_bwd_wt.argtypes = list(L.lyc_lora_linear_bwd.argtypes)
        L.lyc_lora_linear_wc_workspace_size.argtypes = list(L.lyc_lora_linear_workspace_size.argtypes)
        L.lyc_lora_linear_fwd_wc.argtypes = list(L.lyc_lora_linear_fwd.argtypes)
        L.lyc_lora_linear_bwd_saved.argtypes = [c_vp, c_int, c_vp, c_vp, c_int, c_int, c_vp, c_int, c_vp, c_int, c_vp,
                                                c_i64, ctypes.c_double, c_vp, c_int, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                c_i64, c_vp, c_sz, c_vp]
        L.lyc_lora_linear_bwd_workspace_layout.argtypes = [c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int,
                                                           c_int, c_int, c_int, ctypes.POINTER(c_sz),
                                                           ctypes.POINTER(c_sz), ctypes.POINTER(c_i64),
                                                           ctypes.POINTER(c_sz)]
        pi, pd = ctypes.POINTER(c_int), ctypes.POINTER(ctypes.c_double)
        L.lyc_gemm_plan.argtypes = [c_i64, c_i64, c_i64, c_i64, c_int, c_int, pi, pi, pi, pi, pd]
        L.lyc_device_rates.argtypes = [ctypes.POINTER(c_i64), pd, pd, pd, pi]
        L.lyc_measure_device_rates.argtypes = [c_vp]
        L.lyc_lora_linear_tune.argtypes = [c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_i64,
                                           ctypes.c_double, c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_sz, c_vp,
                                           pi, pi, pi, pd, pd]
        L.lyc_tuning_key.argtypes = [c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, c_int, ctypes.c_char_p,
                                     c_sz]
        L.lyc_tuning_lookup.argtypes = [c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, c_int, pi, pi, pi, pi]
        L.lyc_tuning_save.argtypes = [ctypes.c_char_p]
        L.lyc_tuning_load.argtypes = [ctypes.c_char_p, pi]
        L.lyc_tuning_clear.argtypes = []
        L.lyc_tuning_count.argtypes = []
        L.lyc_dora_norms_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_int, c_int, c_int, ctypes.POINTER(c_sz)]
        L.lyc_dora_norms.argtypes = [c_vp, c_int, c_vp, c_int, c_vp, c_int, c_i64, ctypes.c_double, c_vp, c_i64,
                                     c_i64, c_vp, c_sz, c_vp]
        L.lyc_dora_linear_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, c_int,
                                                     c_int, ctypes.POINTER(c_sz)]
        L.lyc_dora_linear_fwd.argtypes = [c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp, c_int, c_vp,
                                          c_int, c_vp, c_i64, ctypes.c_double, c_vp, c_int, c_i64, c_i64, c_i64,
                                          c_vp, c_sz, c_vp]
        L.lyc_gemm_tile.argtypes = [c_i64, c_i64, c_int, ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
        L.lyc_profile_begin.argtypes = [c_int]
        L.lyc_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_int)]
        L.lyc_status_str.argtypes = [c_int]
        L.lyc_status_str.restype = ctypes.c_char_p
        for fn in (L.lyc_resolve_dtypes, L.lyc_linear_workspace_size, L.lyc_linear_fwd, L.lyc_linear_fwd_prepared,
                   L.lyc_linear_prepare,
                   L.lyc_lora_linear_workspace_size, L.lyc_lora_linear_fwd, L.lyc_lora_linear_fwd_noalloc,
                   L.lyc_lora_workspace_layout,
                   L.lyc_linear_workspace_layout, L.lyc_lora_merge_workspace_size, L.lyc_lora_merge_fwd,
                   L.lyc_lora_linear_bwd_workspace_size, L.lyc_lora_linear_bwd, L.lyc_lora_linear_bwd_wt,
                   L.lyc_lora_linear_bwd_saved, L.lyc_lora_linear_wc_workspace_size, L.lyc_lora_linear_fwd_wc,
                   L.lyc_lora_linear_bwd_workspace_layout,
                   L.lyc_gemm_plan, L.lyc_device_rates, L.lyc_measure_device_rates, L.lyc_lora_linear_tune, L.lyc_tuning_key, L.lyc_tuning_lookup, L.lyc_tuning_save,
                   L.lyc_tuning_load, L.lyc_tuning_clear, L.lyc_tuning_count, L.lyc_dora_norms_workspace_size,
                   L.lyc_dora_norms, L.lyc_dora_linear_workspace_size, L.lyc_dora_linear_fwd,
                   L.lyc_gemm_tile, L.lyc_profile_begin, L.lyc_profile_end):
            fn.restype = c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != OK:
        msg = lib().lyc_status_str(status).decode()
        raise (MixedHalfError if status == ERR_MIXED_HALF else LycError)(status, msg)


def dtype_code(t) -> int:
    dt = t.dtype if isinstance(t, torch.Tensor) else t
    if dt not in _CODE:
        raise TypeError(f"unsupported dtype {dt}")
    return _CODE[dt]


def torch_dtype(code: int):
    return _TORCH[code]


def resolve_dtypes(dtypes: Sequence[int]) -> Tuple[int, int]:
    """Dtype policy over the operands' dtype codes -> (compute, output)."""
    arr = (ctypes.c_int * max(1, len(dtypes)))(*dtypes)
    c, o = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().lyc_resolve_dtypes(arr, len(dtypes), ctypes.byref(c), ctypes.byref(o)))
    return c.value, o.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _shape(t: Optional[torch.Tensor], shape, name: str) -> None:
    """Raise ValueError unless t (if given) has exactly this shape.  The C ABI
    takes bare pointers, so a mis-shaped operand would be read (or an output
    written) out of bounds: every shape is checked here before any call."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(s) for s in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(s) for s in shape)}")


def _dims(t: torch.Tensor, n: int, name: str) -> Tuple[int, ...]:
    if t.dim() != n:
        raise ValueError(f"{name} must be {n}-D, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _out_dtype(out: Optional[torch.Tensor], code: int, name: str = "out") -> None:
    if out is not None and out.dtype != _TORCH[code]:
        raise ValueError(f"{name} has dtype {out.dtype}, the dtype policy gives {_TORCH[code]}")


def _lora_shapes(x, w, down, up, bias, out):
    """(M, N, K, r) of a LoRA-bypass call, every operand's shape checked."""
    M, K = _dims(x, 2, "x")
    N, _ = _dims(w, 2, "w")
    r, _ = _dims(down, 2, "down")
    _shape(w, (N, K), "w")
    _shape(down, (r, K), "down")
    _shape(up, (N, r), "up")
    _shape(bias, (N,), "bias")
    _shape(out, (M, N), "out")
    return M, N, K, r


def _need_device(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("lyc operands must be GPU tensors")
        if not t.is_contiguous():
            raise ValueError("lyc operands must be contiguous")
        if t.dtype not in _CODE and t.dtype != torch.uint8:
            raise TypeError(f"unsupported dtype {t.dtype}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("lyc operands must be on one device")
    return dev


def linear_workspace_size(M, N, K, x_dt, w_dt, b_dt=0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().lyc_linear_workspace_size(M, N, K, x_dt, w_dt, b_dt, ctypes.byref(n)))
    return n.value


def lora_workspace_size(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().lyc_lora_linear_workspace_size(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, ctypes.byref(n)))
    return n.value


def lora_workspace_layout(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt):
    """(h_offset, h_ld, flagged_offset, flagged_slots) inside the LoRA
    workspace: the guard's uint32 counts at flagged_offset, flagged_slots of
    them, sum to the number of re-evaluated h elements."""
    ho, ld, fo, ns = ctypes.c_size_t(0), ctypes.c_int64(0), ctypes.c_size_t(0), ctypes.c_int64(0)
    _check(lib().lyc_lora_workspace_layout(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, ctypes.byref(ho),
                                           ctypes.byref(ld), ctypes.byref(fo), ctypes.byref(ns)))
    return ho.value, ld.value, fo.value, ns.value


def linear_workspace_layout(M, N, K, x_dt, w_dt, b_dt=0):
    """(flagged_offset, slots): the guard's per-workgroup uint32 counts inside
    the plain affine workspace (their sum is the re-evaluated count)."""
    fo, ns = ctypes.c_size_t(0), ctypes.c_int64(0)
    _check(lib().lyc_linear_workspace_layout(M, N, K, x_dt, w_dt, b_dt, ctypes.byref(fo), ctypes.byref(ns)))
    return fo.value, ns.value


def lora_merge_workspace_size(N, K, r, w_dt, d_dt, u_dt) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().lyc_lora_merge_workspace_size(N, K, r, w_dt, d_dt, u_dt, ctypes.byref(n)))
    return n.value


BWD_DX, BWD_DDOWN, BWD_DUP, BWD_WT, BWD_H = 1, 2, 4, 8, 16


def lora_bwd_workspace_size(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, dy_dt, want=7) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().lyc_lora_linear_bwd_workspace_size(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, dy_dt, want,
                                                    ctypes.byref(n)))
    return n.value


def lora_bwd_workspace_layout(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, dy_dt, want=7):
    """(h_offset, gh_offset, ld, flagged_offset) inside the backward's workspace
    (an offset of 2^64-1: not computed for this `want`)."""
    ho, go, ld, fo = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_int64(0), ctypes.c_size_t(0)
    _check(lib().lyc_lora_linear_bwd_workspace_layout(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, dy_dt, want,
                                                      ctypes.byref(ho), ctypes.byref(go), ctypes.byref(ld),
                                                      ctypes.byref(fo)))
    return ho.value, go.value, ld.value, fo.value


def gemm_plan(M: int, N: int, K: int, rf: int, compute_dt: int, max_out: int = 7):
    """The tile planner's shortlist, best first: [(tile_n, tile_m, ksplit, modelled_us)]."""
    tn, tm, ks = (ctypes.c_int * 8)(), (ctypes.c_int * 8)(), (ctypes.c_int * 8)()
    cost = (ctypes.c_double * 8)()
    n = ctypes.c_int(0)
    _check(lib().lyc_gemm_plan(M, N, K, rf, compute_dt, max_out, ctypes.byref(n), tn, tm, ks, cost))
    return [(tn[i], tm[i], ks[i], cost[i]) for i in range(n.value)]


def device_rates() -> dict:
    """The planner's model of the current device: CU count, dense MFMA rates
    (16-bit and fp32 operands, flop/s), HBM rate (bytes/s), and whether they
    were measured on it (else MI355X's published peaks per CU)."""
    cus = ctypes.c_int64(0)
    m16, m32, hbm = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    measured = ctypes.c_int(0)
    _check(lib().lyc_device_rates(ctypes.byref(cus), ctypes.byref(m16), ctypes.byref(m32), ctypes.byref(hbm),
                                  ctypes.byref(measured)))
    return {"cus": cus.value, "mfma16_flops": m16.value, "mfma32_flops": m32.value, "hbm_bytes_per_s": hbm.value,
            "measured": bool(measured.value)}


def measure_device_rates(device=None) -> dict:
    """Measure the current (or given) CUDA device's rates for the planner
    (blocks; allocates 512 MiB meanwhile) and return them."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        _check(lib().lyc_measure_device_rates(_stream(dev)))
        return device_rates()


def tuning_cache_path() -> str:
    """Where the tuning table file lives: $LYC_KERNEL_CACHE_DIR/tuning.json
    (default ~/.cache/lyc_kernels)."""
    d = os.environ.get("LYC_KERNEL_CACHE_DIR", os.path.join(os.path.expanduser("~"), ".cache", "lyc_kernels"))
    return os.path.join(d, "tuning.json")


def tuning_save(path: Optional[str] = None) -> str:
    path = path or tuning_cache_path()
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    _check(lib().lyc_tuning_save(path.encode()))
    return path


def tuning_load(path: Optional[str] = None) -> int:
    """Merge a saved table into the process's table; returns the entries read (0 if no file)."""
    path = path or tuning_cache_path()
    if not os.path.exists(path):
        return 0
    n = ctypes.c_int(0)
    _check(lib().lyc_tuning_load(path.encode(), ctypes.byref(n)))
    return n.value


def tuning_clear() -> None:
    _check(lib().lyc_tuning_clear())


def tuning_count() -> int:
    return int(lib().lyc_tuning_count())


def tuning_key(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().lyc_tuning_key(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, buf, 256))
    return buf.value.decode()


def tuning_lookup(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt):
    """(tile_n, tile_m, ksplit) stored for this call on the current device, or None."""
    f, tn, tm, ks = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().lyc_tuning_lookup(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, ctypes.byref(f), ctypes.byref(tn),
                                   ctypes.byref(tm), ctypes.byref(ks)))
    return (tn.value, tm.value, ks.value) if f.value else None


def gemm_tile(M: int, N: int, compute_dt: int) -> Tuple[int, int]:
    """(tile_n, tile_m) of the output tile one workgroup computes for this shape."""
    tn, tm = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().lyc_gemm_tile(M, N, compute_dt, ctypes.byref(tn), ctypes.byref(tm)))
    return tn.value, tm.value


KERNELS = ("cast", "prep", "hpass", "gemm")


def profile_begin(capacity: int) -> None:
    """Record the device time of each following kernel launch (HIP events)."""
    _check(lib().lyc_profile_begin(capacity))


def profile_end():
    """Stop recording; returns {kernel: (launches, total_ms)}."""
    t = (ctypes.c_double * len(KERNELS))()
    n = (ctypes.c_int * len(KERNELS))()
    _check(lib().lyc_profile_end(t, n))
    return {KERNELS[k]: (n[k], t[k]) for k in range(len(KERNELS))}


def _workspace(nbytes: int, dev, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return workspace
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def linear(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           prepared: bool = False) -> torch.Tensor:
    """y = round_out(round_out(x.W^T) + b) on the GPU (plain affine contract).

    ``prepared``: ``workspace`` already holds what the call derives from W
    (``linear_prepare``, or an earlier call with the same W, shapes and
    dtypes), and the call skips those launches."""
    M, K = _dims(x, 2, "x")
    N, _ = _dims(w, 2, "w")
    _shape(w, (N, K), "w")
    _shape(bias, (N,), "bias")
    _shape(out, (M, N), "out")
    x_dt, w_dt = dtype_code(x), dtype_code(w)
    b_dt = dtype_code(bias) if bias is not None else 0
    _, o_dt = resolve_dtypes([x_dt, w_dt] + ([b_dt] if b_dt else []))
    _out_dtype(out, o_dt)
    dev = _need_device(x, w, bias, out, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=_TORCH[o_dt], device=dev)
    if prepared and workspace is None:
        raise ValueError("prepared: pass the prepared workspace")
    ws = _workspace(linear_workspace_size(M, N, K, x_dt, w_dt, b_dt), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    fn = lib().lyc_linear_fwd_prepared if prepared else lib().lyc_linear_fwd
    _check(fn(_ptr(x), x_dt, _ptr(w), w_dt, _ptr(bias), b_dt, _ptr(out), dtype_code(out),
              M, N, K, _ptr(ws), nbytes, _stream(dev)))
    return out


def linear_prepare(w: torch.Tensor, M: int, x_dtype: torch.dtype, bias_dtype: Optional[torch.dtype] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prepare W [N,K] for ``linear(..., prepared=True)`` calls with M token
    rows of dtype ``x_dtype`` (and a bias of ``bias_dtype``): writes W's
    compute-dtype copy (fp32 W) and split into the workspace, which is returned
    (allocated when not given)."""
    N, K = _dims(w, 2, "w")
    x_dt, w_dt = _CODE[x_dtype], dtype_code(w)
    b_dt = _CODE[bias_dtype] if bias_dtype is not None else 0
    dev = _need_device(w, workspace)
    nb = linear_workspace_size(M, N, K, x_dt, w_dt, b_dt)
    ws = workspace if workspace is not None else torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    nbytes = ws.numel() * ws.element_size()
    _check(lib().lyc_linear_prepare(_ptr(w), w_dt, x_dt, b_dt, M, N, K, _ptr(ws), nbytes, _stream(dev)))
    return ws


def lora_linear(x: torch.Tensor, w: torch.Tensor, down: torch.Tensor, up: torch.Tensor, scale: float,
                bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, return_workspace: bool = False,
                w_c: Optional[torch.Tensor] = None):
    """y = round_out(x.W^T + scale * round_c(x.down^T).up^T + b) on the GPU.

    x [M,K], w [N,K], down [r,K], up [N,r], bias [N] (optional).  With
    ``return_workspace`` the workspace tensor is returned too (h_r and the
    guard counter live in it; see ``lora_workspace_layout``).  ``w_c``:
    optional caller-kept copy of W rounded to the compute dtype [N,K] (an
    fp32 W's working copy, made once while W is frozen): the GEMM reads it
    and W is not cast per call; w still sets the dtype policy."""
    M, N, K, r = _lora_shapes(x, w, down, up, bias, out)
    x_dt, w_dt, d_dt, u_dt = dtype_code(x), dtype_code(w), dtype_code(down), dtype_code(up)
    b_dt = dtype_code(bias) if bias is not None else 0
    c_dt, o_dt = resolve_dtypes([x_dt, w_dt] + ([b_dt] if b_dt else []) + [d_dt, u_dt])
    _out_dtype(out, o_dt)
    _shape(w_c, (N, K), "w_c")
    if w_c is not None and w_c.dtype != _TORCH[c_dt]:
        raise ValueError(f"w_c has dtype {w_c.dtype}, the compute dtype is {_TORCH[c_dt]}")
    dev = _need_device(x, w, down, up, bias, out, workspace, w_c)
    if out is None:
        out = torch.empty((M, N), dtype=_TORCH[o_dt], device=dev)
    size = lib().lyc_lora_linear_wc_workspace_size if w_c is not None else lib().lyc_lora_linear_workspace_size
    n = ctypes.c_size_t(0)
    _check(size(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    fn, wp = (lib().lyc_lora_linear_fwd_wc, w_c) if w_c is not None else (lib().lyc_lora_linear_fwd, w)
    _check(fn(_ptr(x), x_dt, _ptr(wp), w_dt, _ptr(bias), b_dt, _ptr(down), d_dt, _ptr(up), u_dt, r, float(scale),
              _ptr(out), dtype_code(out), M, N, K, _ptr(ws), nbytes, _stream(dev)))
    return (out, ws) if return_workspace else out


def lora_linear_noalloc(x: torch.Tensor, w: torch.Tensor, down: torch.Tensor, up: torch.Tensor, scale: float,
                        bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lora_linear through the allocation-free entry point: the library's
    kernels use its static per-GPU scratch array instead of a workspace (for
    callers that cannot allocate device memory; pass ``out`` to allocate
    nothing here either).  Calls that overlap on one GPU race on that array."""
    M, N, K, r = _lora_shapes(x, w, down, up, bias, out)
    x_dt, w_dt, d_dt, u_dt = dtype_code(x), dtype_code(w), dtype_code(down), dtype_code(up)
    b_dt = dtype_code(bias) if bias is not None else 0
    _, o_dt = resolve_dtypes([x_dt, w_dt] + ([b_dt] if b_dt else []) + [d_dt, u_dt])
    _out_dtype(out, o_dt)
    dev = _need_device(x, w, down, up, bias, out)
    if out is None:
        out = torch.empty((M, N), dtype=_TORCH[o_dt], device=dev)
    _check(lib().lyc_lora_linear_fwd_noalloc(_ptr(x), x_dt, _ptr(w), w_dt, _ptr(bias), b_dt, _ptr(down), d_dt,
                                             _ptr(up), u_dt, r, float(scale), _ptr(out), dtype_code(out), M, N, K,
                                             _stream(dev)))
    return out


def lora_merge(w: torch.Tensor, down: torch.Tensor, up: torch.Tensor, scale: float,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W' = round_out(W + scale * up_c.down_c) on the GPU.

    w [N,K], down [r,K], up [N,r].  ``out`` may be ``w`` itself (in-place
    merge, when W already has the output dtype)."""
    N, K = _dims(w, 2, "w")
    r, _ = _dims(down, 2, "down")
    _shape(down, (r, K), "down")
    _shape(up, (N, r), "up")
    _shape(out, (N, K), "out")
    w_dt, d_dt, u_dt = dtype_code(w), dtype_code(down), dtype_code(up)
    _, o_dt = resolve_dtypes([w_dt, d_dt, u_dt])
    _out_dtype(out, o_dt)
    dev = _need_device(w, down, up, out, workspace)
    if out is None:
        out = torch.empty((N, K), dtype=_TORCH[o_dt], device=dev)
    ws = _workspace(lora_merge_workspace_size(N, K, r, w_dt, d_dt, u_dt), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lyc_lora_merge_fwd(_ptr(w), w_dt, _ptr(down), d_dt, _ptr(up), u_dt, r, float(scale), _ptr(out),
                                    dtype_code(out), N, K, _ptr(ws), nbytes, _stream(dev)))
    return out


def lora_saved_h(workspace: torch.Tensor, x: torch.Tensor, w: torch.Tensor, down: torch.Tensor, up: torch.Tensor,
                 bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The h_r [M, r_pad] that lora_linear left in ``workspace`` (returned by
    it with ``return_workspace``) for these operands: a view, valid until the
    workspace is reused; pass it to lora_linear_backward as ``h``."""
    M, N, K, r = _lora_shapes(x, w, down, up, bias, None)
    codes = [dtype_code(t) for t in (x, w)] + [dtype_code(bias) if bias is not None else 0] + \
        [dtype_code(down), dtype_code(up)]
    ho, ld, _, _ = lora_workspace_layout(M, N, K, r, *codes)
    c_dt = resolve_dtypes([c for c in codes if c])[0]
    es = 4 if c_dt == F32 else 2
    return workspace[ho: ho + M * ld * es].view(_TORCH[c_dt]).view(M, ld)


def lora_linear_backward(x: torch.Tensor, w: torch.Tensor, down: torch.Tensor, up: torch.Tensor, scale: float,
                         dy: torch.Tensor, bias_dtype: Optional[torch.dtype] = None, want_dx: bool = True,
                         want_ddown: bool = True, want_dup: bool = True, workspace: Optional[torch.Tensor] = None,
                         return_workspace: bool = False, w_t: Optional[torch.Tensor] = None,
                         h: Optional[torch.Tensor] = None):
    """Gradients (dx, d_down, d_up) of the LoRA-bypass linear for dy, each in
    its leaf's dtype (None where not wanted).  W and the bias are frozen;
    ``bias_dtype`` is the forward's bias dtype (it enters the dtype policy).
    ``w_t``: optional caller-kept W_c^T [K, N] in the compute dtype (W rounded
    to it, then transposed; kept across steps while W is frozen): dx reads it
    in place and no W^T copy is made per call.  ``h``: optional h_r [M, r_pad]
    the forward left (``lora_saved_h``): dUp reads it and no h pass runs."""
    M, N, K, r = _lora_shapes(x, w, down, up, None, None)
    _shape(dy, (M, N), "dy")
    _shape(w_t, (K, N), "w_t")
    dev = _need_device(x, w, down, up, dy, workspace, w_t, h)
    x_dt, w_dt, d_dt, u_dt, g_dt = (dtype_code(t) for t in (x, w, down, up, dy))
    b_dt = dtype_code(torch.empty(0, dtype=bias_dtype)) if bias_dtype is not None else 0
    c_dt = resolve_dtypes([x_dt, w_dt] + ([b_dt] if b_dt else []) + [d_dt, u_dt, g_dt])[0]
    if w_t is not None and w_t.dtype != _TORCH[c_dt]:
        raise ValueError(f"w_t has dtype {w_t.dtype}, the compute dtype is {_TORCH[c_dt]}")
    if h is not None:
        r_pad = lora_bwd_workspace_layout(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, g_dt, BWD_DUP)[2]
        _shape(h, (M, r_pad), "h")
        if h.dtype != _TORCH[c_dt]:
            raise ValueError(f"h has dtype {h.dtype}, the compute dtype is {_TORCH[c_dt]}")
    want = (BWD_DX if want_dx else 0) | (BWD_DDOWN if want_ddown else 0) | (BWD_DUP if want_dup else 0) | \
        (BWD_WT if w_t is not None else 0) | (BWD_H if h is not None else 0)
    dx = torch.empty((M, K), dtype=x.dtype, device=dev) if want_dx else None
    dd = torch.empty((r, K), dtype=down.dtype, device=dev) if want_ddown else None
    du = torch.empty((N, r), dtype=up.dtype, device=dev) if want_dup else None
    ws = _workspace(lora_bwd_workspace_size(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, g_dt, want), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    # an empty output still has to be passed (non-NULL) to be "wanted"
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr() if t.numel() else 256)
    if h is not None:
        _check(lib().lyc_lora_linear_bwd_saved(_ptr(x), x_dt, None if w_t is not None else _ptr(w), _ptr(w_t), w_dt,
                                               b_dt, _ptr(down), d_dt, _ptr(up), u_dt, _ptr(h), r, float(scale),
                                               _ptr(dy), g_dt, p(dx), p(dd), p(du), M, N, K, _ptr(ws), nbytes,
                                               _stream(dev)))
    else:
        fn, wp = (lib().lyc_lora_linear_bwd_wt, w_t) if w_t is not None else (lib().lyc_lora_linear_bwd, w)
        _check(fn(_ptr(x), x_dt, _ptr(wp), w_dt, b_dt, _ptr(down), d_dt, _ptr(up), u_dt, r, float(scale), _ptr(dy),
                  g_dt, p(dx), p(dd), p(du), M, N, K, _ptr(ws), nbytes, _stream(dev)))
    out = (dx, dd, du)
    return (out, ws) if return_workspace else out


def lora_linear_tune(x: torch.Tensor, w: torch.Tensor, down: torch.Tensor, up: torch.Tensor, scale: float,
                     bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """Time the planner's shortlist for this forward (blocking) and keep the
    fastest for later calls of the same shape.  Returns (tile_n, tile_m,
    ksplit, ms, [ms of each shortlisted candidate, in gemm_plan order])."""
    M, N, K, r = _lora_shapes(x, w, down, up, bias, out)
    x_dt, w_dt, d_dt, u_dt = dtype_code(x), dtype_code(w), dtype_code(down), dtype_code(up)
    b_dt = dtype_code(bias) if bias is not None else 0
    _, o_dt = resolve_dtypes([x_dt, w_dt] + ([b_dt] if b_dt else []) + [d_dt, u_dt])
    _out_dtype(out, o_dt)
    dev = _need_device(x, w, down, up, bias, out, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=_TORCH[o_dt], device=dev)
    ws = _workspace(lora_workspace_size(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    tn, tm, ks, ms = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_double(0)
    cand = (ctypes.c_double * 7)(*([-1.0] * 7))
    _check(lib().lyc_lora_linear_tune(_ptr(x), x_dt, _ptr(w), w_dt, _ptr(bias), b_dt, _ptr(down), d_dt, _ptr(up),
                                      u_dt, r, float(scale), _ptr(out), dtype_code(out), M, N, K, _ptr(ws), nbytes,
                                      _stream(dev), ctypes.byref(tn), ctypes.byref(tm), ctypes.byref(ks),
                                      ctypes.byref(ms), cand))
    n = len(gemm_plan(M, N, K, lora_workspace_layout(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt)[1] if r else 0,
                      resolve_dtypes([x_dt, w_dt] + ([b_dt] if b_dt else []) + [d_dt, u_dt])[0]))
    return tn.value, tm.value, ks.value, ms.value, [cand[i] for i in range(n)]


def dora_norms(w: torch.Tensor, down: torch.Tensor, up: torch.Tensor, scale: float,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """DoRA row norms ||W + scale * up_c.down_c||_2 per row of W [N,K], fp32 [N]."""
    N, K = _dims(w, 2, "w")
    r, _ = _dims(down, 2, "down")
    _shape(down, (r, K), "down")
    _shape(up, (N, r), "up")
    _shape(out, (N,), "out")
    _out_dtype(out, F32)
    dev = _need_device(w, down, up, out, workspace)
    w_dt, d_dt, u_dt = dtype_code(w), dtype_code(down), dtype_code(up)
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=dev)
    n = ctypes.c_size_t(0)
    _check(lib().lyc_dora_norms_workspace_size(N, K, r, w_dt, d_dt, u_dt, ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lyc_dora_norms(_ptr(w), w_dt, _ptr(down), d_dt, _ptr(up), u_dt, r, float(scale), _ptr(out), N, K,
                                _ptr(ws), nbytes, _stream(dev)))
    return out


def dora_linear(x: torch.Tensor, w: torch.Tensor, down: torch.Tensor, up: torch.Tensor, scale: float,
                magnitude: torch.Tensor, norms: torch.Tensor, bias: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = round_out((m/norm) * (x.W^T + scale * round_c(x.down^T).up^T) + b) on the GPU."""
    M, N, K, r = _lora_shapes(x, w, down, up, bias, out)
    _shape(magnitude, (N,), "magnitude")
    _shape(norms, (N,), "norms")
    if norms.dtype != torch.float32:
        raise ValueError("DoRA norms are fp32")
    x_dt, w_dt, d_dt, u_dt, m_dt = (dtype_code(t) for t in (x, w, down, up, magnitude))
    b_dt = dtype_code(bias) if bias is not None else 0
    _, o_dt = resolve_dtypes([x_dt, w_dt] + ([b_dt] if b_dt else []) + [d_dt, u_dt, m_dt])
    _out_dtype(out, o_dt)
    dev = _need_device(x, w, down, up, magnitude, norms, bias, out, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=_TORCH[o_dt], device=dev)
    n = ctypes.c_size_t(0)
    _check(lib().lyc_dora_linear_workspace_size(M, N, K, r, x_dt, w_dt, b_dt, d_dt, u_dt, m_dt, ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().lyc_dora_linear_fwd(_ptr(x), x_dt, _ptr(w), w_dt, _ptr(bias), b_dt, _ptr(down), d_dt, _ptr(up), u_dt,
                                     _ptr(magnitude), m_dt, _ptr(norms), r, float(scale), _ptr(out), dtype_code(out),
                                     M, N, K, _ptr(ws), nbytes, _stream(dev)))
    return out
