"""Seeded synthetic workloads for the LoRA-bypass linear.

This module only *draws* inputs: shapes, value distributions and seeds.  It
holds none of the method's arithmetic (no dtype policy, no contraction, no
rounding boundary), so both the GPU path's tests/bench and the CPU oracle can
take their inputs from here without sharing any computation.

Every tensor is drawn from its own counter-based stream: numpy's Philox4x64
keyed by ``(seed, tensor_id)``.  Values are drawn in fp64, converted to fp32
and then to the tensor's storage dtype with torch's round-to-nearest-even
conversion.  The result is a set of CPU tensors; callers copy the identical
bytes to the device.

Distribution notation ``N(mu, v)`` follows the reading that the second
argument is the *variance* (``N(0, 1/768)`` for a 768-wide weight is the
usual 1/fan_in initialisation); standard deviations below are ``sqrt(v)``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Tuple

import numpy as np
import torch

F16, BF16, F32 = 1, 2, 3
TORCH_DTYPE = {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}
NAME = {F16: "f16", BF16: "bf16", F32: "f32"}
BYTES = {F16: 2, BF16: 2, F32: 4}

# tensor ids used to key the per-tensor Philox streams
_TID = {"x": 1, "w": 2, "b": 3, "down": 4, "up": 5, "rowscale": 6, "dy": 7, "magnitude": 8}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic problem: y[M,N] from x[M,K], W[N,K], optional b[N] and,
    for the LoRA form, down[r,K], up[N,r] and scale."""
    name: str
    kind: str                 # "linear" (projection rounded, then + bias) or "lora"
    M: int
    K: int
    N: int
    r: int
    scale: float
    x_dt: int
    w_dt: int                 # dtype of W, down and up (the module weights)
    b_dt: Optional[int]       # None = no bias
    x_std: float
    w_std: float
    down_std: float
    up_std: float
    b_std: float
    row_lognormal: bool       # x rows scaled by exp(N(0,1)) (non-uniform rows)
    seed: int

    def resized(self, M=None, K=None, N=None, r=None, **kw) -> "Workload":
        """Same distributions and dtypes at another size (for parity cases)."""
        d = dataclasses.asdict(self)
        d.update({k: v for k, v in dict(M=M, K=K, N=N, r=r).items() if v is not None})
        d.update(kw)
        return Workload(**d)

    @property
    def flops(self) -> float:
        """Algorithmic flops of one call: 2MNK + 2MKr + 2MrN."""
        return 2.0 * self.M * self.N * self.K + 2.0 * self.M * self.K * self.r + 2.0 * self.M * self.r * self.N

    @property
    def bytes(self) -> float:
        """Algorithmic HBM bytes: every input read once at its stored width, y written once."""
        wb = BYTES[self.w_dt]
        out_dt = self.out_dt_hint
        nb = self.M * self.K * BYTES[self.x_dt] + self.N * self.K * wb
        nb += self.r * self.K * wb + self.N * self.r * wb
        if self.b_dt is not None:
            nb += self.N * BYTES[self.b_dt]
        nb += self.M * self.N * BYTES[out_dt]
        return float(nb)

    @property
    def out_dt_hint(self) -> int:
        """Output storage width used only for the byte count (fp32 if any operand is fp32)."""
        dts = [self.x_dt, self.w_dt] + ([self.b_dt] if self.b_dt is not None else [])
        if F32 in dts:
            return F32
        return self.x_dt if self.x_dt == self.w_dt else F32


def _std(v: float) -> float:
    return math.sqrt(v)


# The five workloads the method is measured on (sizes, dtypes, distributions, seeds).
WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


_add(Workload("affine_f16_1024x768x1024", "linear", M=1024, K=768, N=1024, r=0, scale=0.0,
              x_dt=F16, w_dt=F16, b_dt=F16, x_std=1.0, w_std=_std(1 / 768), down_std=0.0, up_std=0.0,
              b_std=_std(0.1), row_lognormal=False, seed=0))
_add(Workload("lora_f16_4096x3072x3072_r16", "lora", M=4096, K=3072, N=3072, r=16, scale=1.0,
              x_dt=F16, w_dt=F16, b_dt=None, x_std=1.0, w_std=_std(1 / 3072), down_std=_std(1 / 3072),
              up_std=_std(1 / 16), b_std=0.0, row_lognormal=False, seed=1))
_add(Workload("lora_bf16x_f32w_8192x4096x4096_r64", "lora", M=8192, K=4096, N=4096, r=64, scale=0.5,
              x_dt=BF16, w_dt=F32, b_dt=None, x_std=1.0, w_std=_std(1 / 4096), down_std=_std(1 / 4096),
              up_std=_std(1 / 64), b_std=0.0, row_lognormal=False, seed=2))
# dtype-policy sweep: x dtype and module-weight dtype each in {f16, bf16, f32}; bias ~ N(0, 1/fan_in)
for _xd in (F16, BF16, F32):
    for _wd in (F16, BF16, F32):
        _add(Workload(f"sweep_x{NAME[_xd]}_w{NAME[_wd]}_2048x1280x5120_r32", "lora", M=2048, K=1280, N=5120,
                      r=32, scale=1.0, x_dt=_xd, w_dt=_wd, b_dt=_wd, x_std=1.0, w_std=_std(1 / 1280),
                      down_std=_std(1 / 1280), up_std=_std(1 / 32), b_std=_std(1 / 1280),
                      row_lognormal=False, seed=3))
_add(Workload("lora_bf16_16384x8192x8192_r128", "lora", M=16384, K=8192, N=8192, r=128, scale=2.0,
              x_dt=BF16, w_dt=BF16, b_dt=BF16, x_std=1.0, w_std=_std(1 / 8192), down_std=_std(1 / 8192),
              up_std=_std(1 / 128), b_std=_std(0.1), row_lognormal=True, seed=4))

SWEEP = [n for n in WORKLOADS if n.startswith("sweep_")]


def _stream(seed: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=np.array([seed, _TID[tensor]], dtype=np.uint64)))


def _draw(seed: int, tensor: str, shape: Tuple[int, ...], std: float, dt: int) -> torch.Tensor:
    n = int(np.prod(shape)) if len(shape) else 1
    a = _stream(seed, tensor).standard_normal(n) * std
    t = torch.from_numpy(a.astype(np.float32).reshape(shape))
    return t.to(TORCH_DTYPE[dt]).contiguous()


def generate(w: Workload) -> Dict[str, torch.Tensor]:
    """Draw the inputs of ``w`` as CPU tensors in their storage dtypes.

    Returns a dict with x [M,K], w [N,K], b [N] (if any), down [r,K] and
    up [N,r] (LoRA form).  Row-scaled x: s_m = exp(N(0,1)) per row, then
    x[m,:] = s_m * z[m,:] with z ~ N(0, x_std^2)."""
    out: Dict[str, torch.Tensor] = {}
    if w.row_lognormal:
        s = np.exp(_stream(w.seed, "rowscale").standard_normal(w.M))
        z = _stream(w.seed, "x").standard_normal(w.M * w.K).reshape(w.M, w.K) * w.x_std
        z *= s[:, None]
        out["x"] = torch.from_numpy(z.astype(np.float32)).to(TORCH_DTYPE[w.x_dt]).contiguous()
        del z
    else:
        out["x"] = _draw(w.seed, "x", (w.M, w.K), w.x_std, w.x_dt)
    out["w"] = _draw(w.seed, "w", (w.N, w.K), w.w_std, w.w_dt)
    if w.b_dt is not None:
        out["b"] = _draw(w.seed, "b", (w.N,), w.b_std, w.b_dt)
    if w.kind == "lora":
        out["down"] = _draw(w.seed, "down", (w.r, w.K), w.down_std, w.w_dt)
        out["up"] = _draw(w.seed, "up", (w.N, w.r), w.up_std, w.w_dt)
    return out


def generate_dy(w: Workload, dt: int, std: float = 1.0) -> torch.Tensor:
    """The upstream gradient dy [M,N] for the backward: N(0, std^2) in dtype dt
    (the forward's output dtype), from its own Philox stream."""
    return _draw(w.seed, "dy", (w.M, w.N), std, dt)


def generate_magnitude(w: Workload) -> torch.Tensor:
    """A DoRA magnitude vector m [N]: N(1, 0.1^2) in the module weights' dtype
    (the row norms of a 1/fan_in-initialised W are close to 1)."""
    a = 1.0 + 0.1 * _stream(w.seed, "magnitude").standard_normal(w.N)
    return torch.from_numpy(a.astype(np.float32)).to(TORCH_DTYPE[w.w_dt]).contiguous()


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """The stored bytes of a CPU tensor as a numpy array (uint16 for 16-bit, float32 for fp32)."""
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.contiguous().numpy()
    raise TypeError(t.dtype)


def digest(tensors: Dict[str, torch.Tensor]) -> str:
    """sha256 over the stored bytes of every tensor, in key order (recorded with results)."""
    h = hashlib.sha256()
    for k in sorted(tensors):
        h.update(k.encode())
        h.update(raw_bits(tensors[k]).tobytes())
    return h.hexdigest()[:16]


def dtype_code(t: torch.Tensor) -> int:
    return {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}[t.dtype]
