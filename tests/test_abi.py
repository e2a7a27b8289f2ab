"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/lyc.h declares, resolves the dtype policy exactly, and refuses bad
arguments with the documented codes before any GPU work (fake pointers are
never dereferenced because every check precedes the first launch)."""
import ctypes
import itertools
import os
import re

import pytest
import torch

import lora_bypass_linear_amd as L
import oracle
from tests import exact

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lyc.h")
V = ctypes.c_void_p
P = V(4096)            # a fake, 256-aligned "device pointer" that is never touched


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lyc_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 7, names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), f"liblyc.so does not export {n}"


def test_status_strings():
    lib = L.lib()
    for s in range(9):
        assert lib.lyc_status_str(s) != b"unknown status"
    assert lib.lyc_status_str(99) == b"unknown status"


def test_policy_table_through_abi():
    for x_dt, w_dt, c_dt, o_dt in exact.load_policy_table():
        if c_dt is None:
            with pytest.raises(L.MixedHalfError):
                L.resolve_dtypes([x_dt, w_dt, w_dt, w_dt, w_dt])
        else:
            assert L.resolve_dtypes([x_dt, w_dt, w_dt, w_dt, w_dt]) == (c_dt, o_dt)


def test_policy_matches_oracle_on_every_tuple():
    for n in range(1, 6):
        for tup in itertools.product([1, 2, 3], repeat=n):
            st, c, o = oracle.resolve(list(tup))
            if st == oracle.MIXED_HALF:
                with pytest.raises(L.MixedHalfError):
                    L.resolve_dtypes(list(tup))
            else:
                assert L.resolve_dtypes(list(tup)) == (c, o), tup


# The pointers below are fake: every call must be refused by the argument
# checks (or be an empty no-op) so that nothing is ever launched with them.
def _refused(st, allow_ok=False):
    assert st != L.ERR_HIP and (allow_ok or st != L.OK), f"call was not refused before launching (status {st})"
    return st


def _lin(allow_ok=False, **kw):
    a = dict(x=P, x_dt=1, w=P, w_dt=1, b=None, b_dt=0, y=P, y_dt=1, M=4, N=4, K=8, ws=None, nws=0, s=None)
    a.update(kw)
    return _refused(L.lib().lyc_linear_fwd(a["x"], a["x_dt"], a["w"], a["w_dt"], a["b"], a["b_dt"], a["y"],
                                           a["y_dt"], a["M"], a["N"], a["K"], a["ws"], a["nws"], a["s"]), allow_ok)


def _lora(allow_ok=False, **kw):
    a = dict(x=P, x_dt=1, w=P, w_dt=1, b=None, b_dt=0, d=P, d_dt=1, u=P, u_dt=1, r=4, scale=1.0, y=P, y_dt=1,
             M=4, N=4, K=8, ws=None, nws=0, s=None)
    a.update(kw)
    return _refused(L.lib().lyc_lora_linear_fwd(a["x"], a["x_dt"], a["w"], a["w_dt"], a["b"], a["b_dt"], a["d"],
                                                a["d_dt"], a["u"], a["u_dt"], a["r"], ctypes.c_double(a["scale"]),
                                                a["y"], a["y_dt"], a["M"], a["N"], a["K"], a["ws"], a["nws"], a["s"]),
                    allow_ok)


def test_linear_argument_errors():
    assert _lin(w_dt=2) == L.ERR_MIXED_HALF
    assert _lin(y_dt=3) == L.ERR_DTYPE_MISMATCH
    assert _lin(x_dt=3, y_dt=1) == L.ERR_DTYPE_MISMATCH      # fp32 x promotes the output to fp32
    assert _lin(x_dt=7) == L.ERR_INVALID_ARG
    assert _lin(M=-1) == L.ERR_INVALID_ARG
    assert _lin(K=12) == L.ERR_UNSUPPORTED                   # rows must be 16-byte multiples
    assert _lin(x=V(4098)) == L.ERR_UNSUPPORTED              # misaligned x
    assert _lin(x=None) == L.ERR_INVALID_ARG
    assert _lin(y=None) == L.ERR_INVALID_ARG
    assert _lin(b=P, b_dt=0) == L.ERR_INVALID_ARG             # bias pointer without a dtype
    assert _lin(b=None, b_dt=1) == L.ERR_INVALID_ARG          # dtype without a bias
    assert _lin(b=P, b_dt=2) == L.ERR_MIXED_HALF
    # an fp16 bias counts as a 16-bit operand: compute fp16 (fp32 x and W need fp16 copies), output fp32
    assert _lin(x_dt=3, w_dt=3, y_dt=1, b=P, b_dt=1) == L.ERR_DTYPE_MISMATCH
    assert _lin(x_dt=3, w_dt=3, y_dt=3, b=P, b_dt=1) == L.ERR_WORKSPACE
    # the projection guard (and fp16 copies of fp32 operands) need a workspace
    assert _lin() == L.ERR_WORKSPACE
    assert _lin(w_dt=3, y_dt=3) == L.ERR_WORKSPACE
    assert _lin(w_dt=3, y_dt=3, ws=V(4100), nws=1 << 20) == L.ERR_WORKSPACE   # not 256-aligned


def test_empty_calls_are_noops():
    # nothing is launched for an empty output, so null data pointers are fine
    assert _lin(M=0, x=None, y=None, allow_ok=True) == L.OK
    assert _lin(N=0, w=None, y=None, allow_ok=True) == L.OK
    assert _lora(M=0, x=None, y=None, allow_ok=True) == L.OK


def test_lora_argument_errors():
    assert _lora(d_dt=2) == L.ERR_MIXED_HALF
    assert _lora(r=257) == L.ERR_UNSUPPORTED                  # rank beyond the kernel budget
    assert _lora(r=-1) == L.ERR_INVALID_ARG
    assert _lora(u=None) == L.ERR_INVALID_ARG
    assert _lora(d=None) == L.ERR_INVALID_ARG
    assert _lora() == L.ERR_WORKSPACE
    assert _lora(ws=P, nws=16) == L.ERR_WORKSPACE
    assert _lora(scale=float("nan")) == L.ERR_INVALID_ARG
    assert _lora(scale=float("inf")) == L.ERR_INVALID_ARG
    assert _lora(y_dt=2) == L.ERR_DTYPE_MISMATCH               # y is not a policy operand: bf16 y for fp16 operands
    assert _lora(u_dt=3, y_dt=1) == L.ERR_DTYPE_MISMATCH


def test_workspace_sizes():
    # LoRA workspace = h [M, r_pad] + down/up copies + norms + counter (+ casts of fp32 x/W)
    n16 = L.lora_workspace_size(1000, 300, 64, 17, 1, 1, 0, 1, 1)
    assert n16 >= 1000 * 32 * 2 + 32 * 64 * 2 + 300 * 32 * 2 + 32 * 8
    ho, ld, fo, ns = L.lora_workspace_layout(1000, 300, 64, 17, 1, 1, 0, 1, 1)
    assert ld == 32 and ho % 256 == 0 and fo % 256 == 0 and ns == 1 and fo + 4 * ns <= n16
    # few token rows: h one fp64 dot per element, one guard count per workgroup of 4 waves
    n_small = L.lora_workspace_size(16, 3072, 3072, 16, 1, 1, 0, 1, 1)
    ho, ld, fo, ns = L.lora_workspace_layout(16, 3072, 3072, 16, 1, 1, 0, 1, 1)
    assert ld == 16 and ns == 16 * 16 // 4 and fo + 4 * ns <= n_small
    # above 128 rows: the split form; at rank 16 with down in the compute dtype
    # it splits down itself and counts per workgroup (16 rows each, 8 k groups
    # up to 4096 rows; 32 rows, 2 k groups, from 8192)
    assert L.lora_workspace_layout(129, 3072, 3072, 16, 1, 1, 0, 1, 1)[3] == 9
    assert L.lora_workspace_layout(4096, 3072, 3072, 16, 1, 1, 0, 1, 1)[3] == 256
    assert L.lora_workspace_layout(16384, 3072, 3072, 16, 2, 2, 0, 2, 2)[3] == 512
    assert L.lora_workspace_layout(4096, 3072, 3072, 16, 1, 1, 0, 3, 1)[3] == 1   # fp32 down: prepared, one counter
    assert L.lora_workspace_layout(4096, 3072, 3072, 12, 1, 1, 0, 1, 1)[3] == 1   # rank padded to 16: prepared
    assert L.lora_workspace_layout(128, 8192, 8192, 128, 2, 2, 0, 2, 2)[3] == 1   # M r_pad K above 2^25
    # affine: one guard count per workgroup of the contraction (+ a bf16 copy of an fp32 W)
    fo, ns = L.linear_workspace_layout(64, 64, 64, 1, 1)
    assert ns >= 1 and L.linear_workspace_size(64, 64, 64, 1, 1) >= fo + 4 * ns
    assert L.linear_workspace_layout(1024, 1024, 768, 1, 1)[1] == 256         # 64 x 64 tiles: W split beforehand
    assert L.linear_workspace_layout(1000, 1100, 768, 1, 1)[1] == 16 * 18     # (ragged: tiles over M and N)
    assert L.linear_workspace_size(1024, 1024, 768, 1, 1) >= 2 * 1024 * 768 * 2
    assert L.linear_workspace_layout(16, 1024, 768, 1, 1)[1] == 64            # 16 x 16 workgroups, 8 k groups
    assert L.linear_workspace_layout(256, 512, 768, 1, 1)[1] == 8 * 32        # 32-row workgroups, 2 k groups
    assert L.linear_workspace_size(64, 32, 64, 2, 3) >= 32 * 64 * 2
    assert L.linear_workspace_layout(64, 32, 64, 3, 3)[1] == 0                # fp32 compute: no guard
    assert L.lora_workspace_size(8, 8, 8, 0, 1, 1, 0, 1, 1) == 0        # rank 0: no bypass
    for r, pad in ((1, 16), (16, 16), (17, 32), (32, 32), (33, 64), (64, 64), (65, 128), (129, 256), (256, 256)):
        assert L.lora_workspace_layout(16, 16, 16, r, 2, 2, 0, 2, 2)[1] == pad
    # fp32 compute pads small ranks to 32
    assert L.lora_workspace_layout(16, 16, 16, 8, 3, 3, 0, 3, 3)[1] == 32


def _merge(allow_ok=False, **kw):
    a = dict(w=P, w_dt=1, d=P, d_dt=1, u=P, u_dt=1, r=4, scale=1.0, o=V(1 << 30), o_dt=1, N=64, K=64, ws=None,
             nws=0, s=None)
    a.update(kw)
    return _refused(L.lib().lyc_lora_merge_fwd(a["w"], a["w_dt"], a["d"], a["d_dt"], a["u"], a["u_dt"], a["r"],
                                               ctypes.c_double(a["scale"]), a["o"], a["o_dt"], a["N"], a["K"],
                                               a["ws"], a["nws"], a["s"]), allow_ok)


def test_merge_argument_errors():
    assert _merge(d_dt=2) == L.ERR_MIXED_HALF
    assert _merge(w_dt=2) == L.ERR_MIXED_HALF
    assert _merge(o_dt=2) == L.ERR_DTYPE_MISMATCH
    assert _merge(w_dt=3, o_dt=1) == L.ERR_DTYPE_MISMATCH     # an fp32 W promotes W' to fp32
    assert _merge(r=257) == L.ERR_UNSUPPORTED
    assert _merge(r=-1) == L.ERR_INVALID_ARG
    assert _merge(N=-1) == L.ERR_INVALID_ARG
    assert _merge(N=1 << 20, K=1 << 20) == L.ERR_UNSUPPORTED  # more elements than one GPU holds
    assert _merge(w_dt=9) == L.ERR_INVALID_ARG
    assert _merge(scale=float("nan")) == L.ERR_INVALID_ARG
    assert _merge(scale=1e39) == L.ERR_INVALID_ARG
    assert _merge(w=None) == L.ERR_INVALID_ARG
    assert _merge(o=None) == L.ERR_INVALID_ARG
    assert _merge(u=None) == L.ERR_INVALID_ARG
    assert _merge(d=None) == L.ERR_INVALID_ARG
    # W' may be W itself, but may not overlap it otherwise
    assert _merge(o=V(4096 + 128)) == L.ERR_INVALID_ARG
    assert _merge(w=V(1 << 20), o=V((1 << 20) - 64 * 64 * 2 + 2)) == L.ERR_INVALID_ARG
    assert _merge(w_dt=3, d_dt=3, u_dt=1, o=P, o_dt=3) == L.ERR_WORKSPACE   # in place passes the overlap check
    assert _merge(w=V(4097)) == L.ERR_UNSUPPORTED             # W not element-aligned
    assert _merge(o=V((1 << 30) + 1)) == L.ERR_UNSUPPORTED
    assert _merge() == L.ERR_WORKSPACE
    assert _merge(ws=V(4100), nws=1 << 20) == L.ERR_WORKSPACE
    assert _merge(ws=P, nws=16) == L.ERR_WORKSPACE
    # empty merges launch nothing
    assert _merge(N=0, w=None, o=None, allow_ok=True) == L.OK
    assert _merge(K=0, w=None, o=None, allow_ok=True) == L.OK


def test_merge_workspace_sizes():
    # down^T_c [K][r_pad] + up_c [N][r_pad], each 256-aligned; none without a rank
    assert L.lora_merge_workspace_size(300, 64, 17, 1, 1, 1) == 64 * 32 * 2 + 300 * 32 * 2 + (-(300 * 32 * 2) % 256)
    assert L.lora_merge_workspace_size(64, 64, 8, 3, 3, 3) == 64 * 16 * 4 * 2
    assert L.lora_merge_workspace_size(64, 64, 8, 3, 2, 3) == 64 * 16 * 2 * 2   # bf16 compute copies
    assert L.lora_merge_workspace_size(64, 64, 0, 1, 1, 1) == 0
    with pytest.raises(L.MixedHalfError):
        L.lora_merge_workspace_size(64, 64, 4, 1, 2, 1)


def _bwd(allow_ok=False, **kw):
    a = dict(x=P, x_dt=1, w=P, w_dt=1, b_dt=0, d=P, d_dt=1, u=P, u_dt=1, r=4, scale=1.0, g=P, g_dt=1,
             dx=V(1 << 30), dd=V(1 << 31), du=V(1 << 32), M=16, N=16, K=16, ws=None, nws=0, s=None)
    a.update(kw)
    return _refused(L.lib().lyc_lora_linear_bwd(a["x"], a["x_dt"], a["w"], a["w_dt"], a["b_dt"], a["d"], a["d_dt"],
                                                a["u"], a["u_dt"], a["r"], ctypes.c_double(a["scale"]), a["g"],
                                                a["g_dt"], a["dx"], a["dd"], a["du"], a["M"], a["N"], a["K"],
                                                a["ws"], a["nws"], a["s"]), allow_ok)


def test_backward_argument_errors():
    assert _bwd(g_dt=2) == L.ERR_MIXED_HALF                  # dy is a policy operand
    assert _bwd(b_dt=2) == L.ERR_MIXED_HALF                  # so is the forward's bias dtype
    assert _bwd(K=12) == L.ERR_UNSUPPORTED
    assert _bwd(N=12) == L.ERR_UNSUPPORTED                   # N is a contraction length here
    assert _bwd(M=(1 << 20) + 8) == L.ERR_UNSUPPORTED
    assert _bwd(r=257) == L.ERR_UNSUPPORTED
    assert _bwd(r=-1) == L.ERR_INVALID_ARG
    assert _bwd(x_dt=5) == L.ERR_INVALID_ARG
    assert _bwd(scale=float("nan")) == L.ERR_INVALID_ARG
    assert _bwd(g=None) == L.ERR_INVALID_ARG
    assert _bwd(x=None) == L.ERR_INVALID_ARG
    assert _bwd(u=None) == L.ERR_INVALID_ARG
    assert _bwd(x=V(4096 + 2)) == L.ERR_UNSUPPORTED           # x read in place: 16-byte rows
    assert _bwd(g=V(4096 + 2)) == L.ERR_UNSUPPORTED
    assert _bwd(dx=V(4096 + 256)) == L.ERR_INVALID_ARG        # dx overlaps the inputs
    assert _bwd(dd=V(1 << 30)) == L.ERR_INVALID_ARG           # two gradients overlap
    assert _bwd(dx=V((1 << 30) + 1)) == L.ERR_UNSUPPORTED      # element alignment
    assert _bwd() == L.ERR_WORKSPACE
    assert _bwd(ws=V(4100), nws=1 << 30) == L.ERR_WORKSPACE


def test_backward_workspace_sizes():
    n_all = L.lora_bwd_workspace_size(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 7)
    n_dx = L.lora_bwd_workspace_size(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 1)
    n_du = L.lora_bwd_workspace_size(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 4)
    # dx needs W^T [K][N], down^T [K][32] and gh [M][32]; under 16-bit compute dUp reads dy as
    # stored and needs h [M][32] (and down_c for it), no dy^T [N][M8]
    assert n_dx >= 128 * 64 * 2 + 128 * 32 * 2 + 300 * 32 * 2
    # h [M][32] + down_c with its two splits + up_c + norms: room for no dy^T copy (64 * 304 * 2)
    assert 300 * 32 * 2 <= n_du < 300 * 32 * 2 + 4 * 128 * 32 * 2 + 64 * 32 * 2 + 2048
    assert n_all >= max(n_dx, n_du)
    # fp32 compute: transposed copies, W^T [K][N] for dx and dy^T [N][M8] with h^T for dUp
    n_dx32 = L.lora_bwd_workspace_size(300, 64, 128, 17, 3, 3, 0, 3, 3, 3, 1)
    n_du32 = L.lora_bwd_workspace_size(300, 64, 128, 17, 3, 3, 0, 3, 3, 3, 4)
    assert n_dx32 >= 128 * 64 * 4 + 300 * 32 * 4 and n_du32 >= 64 * 304 * 4 + 32 * 304 * 4
    ho, go, ld, fo = L.lora_bwd_workspace_layout(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 1)
    assert ho == 2 ** 64 - 1 and go % 256 == 0 and ld == 32      # dx alone recomputes no h
    ho, go, ld, fo = L.lora_bwd_workspace_layout(300, 64, 128, 17, 3, 3, 0, 3, 3, 3, 7)
    assert ho % 256 == 0 and fo == 2 ** 64 - 1                    # fp32 compute: no guard
    with pytest.raises(L.MixedHalfError):
        L.lora_bwd_workspace_size(8, 8, 8, 2, 1, 1, 0, 1, 1, 2, 7)


def test_dora_argument_errors():
    lib = L.lib()
    n = ctypes.c_size_t(0)
    assert lib.lyc_dora_norms_workspace_size(64, 64, 4, 1, 1, 1, ctypes.byref(n)) == L.OK and n.value > 0
    assert lib.lyc_dora_norms_workspace_size(64, 64, 4, 1, 2, 1, ctypes.byref(n)) == L.ERR_MIXED_HALF
    args = lambda **kw: {**dict(w=P, w_dt=1, d=P, d_dt=1, u=P, u_dt=1, r=4, s=ctypes.c_double(1.0),
                                o=V(1 << 30), N=64, K=64, ws=None, nws=0, st=None), **kw}
    call = lambda a: _refused(lib.lyc_dora_norms(a["w"], a["w_dt"], a["d"], a["d_dt"], a["u"], a["u_dt"], a["r"],
                                                 a["s"], a["o"], a["N"], a["K"], a["ws"], a["nws"], a["st"]))
    assert call(args()) == L.ERR_WORKSPACE
    assert call(args(o=None)) == L.ERR_INVALID_ARG
    assert call(args(o=V(4096 + 64))) == L.ERR_INVALID_ARG           # norms overlap W
    assert call(args(r=300)) == L.ERR_UNSUPPORTED
    assert call(args(s=ctypes.c_double(float("inf")))) == L.ERR_INVALID_ARG
    # the forward: the magnitude's dtype is a policy operand and is required
    assert lib.lyc_dora_linear_workspace_size(8, 8, 8, 2, 1, 1, 0, 1, 1, 2, ctypes.byref(n)) == L.ERR_MIXED_HALF
    assert lib.lyc_dora_linear_workspace_size(8, 8, 8, 2, 1, 1, 0, 1, 1, 0, ctypes.byref(n)) == L.ERR_INVALID_ARG
    base = L.lora_workspace_size(8, 8, 8, 2, 1, 1, 0, 1, 1)
    assert lib.lyc_dora_linear_workspace_size(8, 8, 8, 2, 1, 1, 0, 1, 1, 1, ctypes.byref(n)) == L.OK
    assert n.value >= base + 8 * 4                                     # plus the gain vector
    f = lambda **kw: _refused(lib.lyc_dora_linear_fwd(
        P, 1, P, 1, None, 0, P, 1, P, 1, kw.get("m", P), 1, kw.get("nm", P), 2, ctypes.c_double(1.0),
        V(1 << 30), kw.get("y_dt", 1), 8, 8, 8, None, 0, None))
    assert f(m=None) == L.ERR_INVALID_ARG and f(nm=None) == L.ERR_INVALID_ARG
    assert f(y_dt=3) == L.ERR_DTYPE_MISMATCH
    assert f(nm=V(4098)) == L.ERR_UNSUPPORTED
    assert f() == L.ERR_WORKSPACE


# ---- the binding checks every operand's shape (and out's dtype) before any call -----

def _t(*shape, dt=torch.float16):
    return torch.zeros(shape, dtype=dt)


@pytest.mark.parametrize("case", [
    dict(w=(64, 40)),            # W's K differs from x's
    dict(down=(8, 40)),          # down's K
    dict(up=(8, 64)),            # up passed as [r, N]
    dict(up=(64, 4)),            # up's rank differs from down's
    dict(bias=(63,)),            # bias length
    dict(out=(32, 63)),          # out shape
    dict(x=(32, 48, 1)),         # x not 2-D
])
def test_binding_rejects_misshaped_lora_operands(case):
    shapes = dict(x=(32, 48), w=(64, 48), down=(8, 48), up=(64, 8), bias=(64,), out=(32, 64))
    shapes.update(case)
    ts = {k: _t(*v) for k, v in shapes.items()}
    with pytest.raises(ValueError, match="shape|-D"):
        L.lora_linear(ts["x"], ts["w"], ts["down"], ts["up"], 1.0, ts["bias"], out=ts["out"])
    if "bias" not in case and "out" not in case:
        with pytest.raises(ValueError, match="shape|-D"):
            L.lora_linear_backward(ts["x"], ts["w"], ts["down"], ts["up"], 1.0, _t(32, 64))
        with pytest.raises(ValueError, match="shape|-D"):
            L.dora_linear(ts["x"], ts["w"], ts["down"], ts["up"], 1.0, _t(64), _t(64, dt=torch.float32))


def test_binding_rejects_misshaped_other_operands():
    x, w = _t(32, 48), _t(64, 48)
    with pytest.raises(ValueError, match="shape"):
        L.linear(x, _t(64, 40))
    with pytest.raises(ValueError, match="shape"):
        L.linear(x, w, _t(60))
    with pytest.raises(ValueError, match="shape"):
        L.linear(x, w, out=_t(32, 60))
    with pytest.raises(ValueError, match="dtype"):
        L.linear(x, w, out=_t(32, 64, dt=torch.bfloat16))                 # the policy gives fp16
    with pytest.raises(ValueError, match="shape"):
        L.lora_merge(w, _t(8, 40), _t(64, 8), 1.0)
    with pytest.raises(ValueError, match="shape"):
        L.lora_merge(w, _t(8, 48), _t(8, 64), 1.0)
    with pytest.raises(ValueError, match="shape"):
        L.lora_merge(w, _t(8, 48), _t(64, 8), 1.0, out=_t(48, 64))              # in-place view of the wrong shape
    with pytest.raises(ValueError, match="dtype"):
        L.lora_merge(w, _t(8, 48), _t(64, 8), 1.0, out=_t(64, 48, dt=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        L.lora_linear_backward(x, w, _t(8, 48), _t(64, 8), 1.0, _t(64, 32))   # dy transposed
    with pytest.raises(ValueError, match="shape"):
        L.dora_norms(w, _t(8, 48), _t(64, 8), 1.0, out=_t(63, dt=torch.float32))
    with pytest.raises(ValueError, match="dtype"):
        L.dora_norms(w, _t(8, 48), _t(64, 8), 1.0, out=_t(64))
    with pytest.raises(ValueError, match="shape"):
        L.dora_linear(x, w, _t(8, 48), _t(64, 8), 1.0, _t(60), _t(64, dt=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        L.lora_linear_tune(x, w, _t(8, 48), _t(8, 64), 1.0)
    # well-shaped CPU operands get past the shape checks and are refused as host memory
    with pytest.raises(ValueError, match="GPU"):
        L.lora_linear(x, w, _t(8, 48), _t(64, 8), 1.0, _t(64))


def test_noalloc_refuses_before_any_gpu_call():
    """The allocation-free forward checks the problem and its scratch need
    before it touches the GPU (fake pointers: nothing is dereferenced)."""
    lib = L.lib()
    call = lambda **kw: lib.lyc_lora_linear_fwd_noalloc(*[{**dict(
        x=P, x_dt=1, w=P, w_dt=1, b=None, b_dt=0, d=P, d_dt=1, u=P, u_dt=1, r=16, scale=ctypes.c_double(1.0), y=P,
        y_dt=1, M=64, N=64, K=64, s=None), **kw}[k] for k in ("x", "x_dt", "w", "w_dt", "b", "b_dt", "d", "d_dt", "u",
                                                              "u_dt", "r", "scale", "y", "y_dt", "M", "N", "K", "s")])
    assert call(w_dt=2) == L.ERR_MIXED_HALF
    assert call(K=12) == L.ERR_UNSUPPORTED
    assert call(r=-1) == L.ERR_INVALID_ARG
    # scratch need beyond the static array: bf16 x with fp32 weights keeps a bf16 copy of W (128 MiB here)
    need = L.lora_workspace_size(16384, 8192, 8192, 128, 2, 3, 0, 3, 3)
    assert need > L.NOALLOC_SCRATCH_BYTES
    assert call(M=16384, N=8192, K=8192, r=128, x_dt=2, w_dt=3, d_dt=3, u_dt=3, y_dt=3) == L.ERR_SCRATCH
    assert b"allocation-free" in lib.lyc_status_str(L.ERR_SCRATCH)
    # the largest workload's need fits
    assert L.lora_workspace_size(16384, 8192, 8192, 128, 2, 2, 2, 2, 2) <= L.NOALLOC_SCRATCH_BYTES


def test_backward_with_caller_kept_wt_checks():
    """lyc_lora_linear_bwd_wt: W^T read in place (16-byte aligned, no overlap
    with an output) and no W^T copy in the workspace (want bit 8)."""
    lib = L.lib()
    a = dict(x=P, x_dt=1, wt=V(1 << 28), w_dt=1, b_dt=0, d=P, d_dt=1, u=P, u_dt=1, r=4, scale=1.0, g=P, g_dt=1,
             dx=V(1 << 30), dd=V(1 << 31), du=V(1 << 32), M=16, N=64, K=64, ws=None, nws=0, s=None)
    call = lambda **kw: _refused(lib.lyc_lora_linear_bwd_wt(*[{**a, **kw}[k] for k in (
        "x", "x_dt", "wt", "w_dt", "b_dt", "d", "d_dt", "u", "u_dt", "r")], ctypes.c_double({**a, **kw}["scale"]),
        *[{**a, **kw}[k] for k in ("g", "g_dt", "dx", "dd", "du", "M", "N", "K", "ws", "nws", "s")]))
    assert call(wt=None) == L.ERR_INVALID_ARG
    assert call(wt=V((1 << 28) + 8)) == L.ERR_UNSUPPORTED        # W^T rows are read 16 bytes at a time
    assert call(wt=V(1 << 30)) == L.ERR_INVALID_ARG              # overlaps dx
    assert call(g_dt=2) == L.ERR_MIXED_HALF
    assert call() == L.ERR_WORKSPACE
    full = L.lora_bwd_workspace_size(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 7)
    kept = L.lora_bwd_workspace_size(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 7 | 8)
    assert full - kept == 128 * 64 * 2                           # exactly the W^T [K][N] copy
    with pytest.raises(L.LycError):
        L.lora_bwd_workspace_size(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 32)


def test_backward_with_saved_h_checks():
    """lyc_lora_linear_bwd_saved: at most one of W and W^T, h_r read in place
    (16-byte aligned, no overlap with an output), and no h pass's regions in
    the workspace (want bit 16)."""
    lib = L.lib()
    a = dict(x=P, x_dt=1, w=P, wt=None, w_dt=1, b_dt=0, d=P, d_dt=1, u=P, u_dt=1, h=V(1 << 29), r=4, scale=1.0,
             g=P, g_dt=1, dx=V(1 << 30), dd=V(1 << 31), du=V(1 << 32), M=16, N=64, K=64, ws=None, nws=0, s=None)
    call = lambda **kw: _refused(lib.lyc_lora_linear_bwd_saved(*[{**a, **kw}[k] for k in (
        "x", "x_dt", "w", "wt", "w_dt", "b_dt", "d", "d_dt", "u", "u_dt", "h", "r")],
        ctypes.c_double({**a, **kw}["scale"]),
        *[{**a, **kw}[k] for k in ("g", "g_dt", "dx", "dd", "du", "M", "N", "K", "ws", "nws", "s")]))
    assert call(wt=V(1 << 28)) == L.ERR_INVALID_ARG               # W and W^T both given
    assert call(h=V((1 << 29) + 8)) == L.ERR_UNSUPPORTED           # h_r rows are read 16 bytes at a time
    assert call(h=V(1 << 32)) == L.ERR_INVALID_ARG                 # overlaps dUp
    assert call(g_dt=2) == L.ERR_MIXED_HALF
    assert call() == L.ERR_WORKSPACE
    assert call(h=None) == L.ERR_WORKSPACE                         # no h_r: recomputed, as lyc_lora_linear_bwd
    full = L.lora_bwd_workspace_size(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 7)
    saved = L.lora_bwd_workspace_size(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 7 | 16)
    # the h pass's regions (rank 17 pads to 32): down_c and its hi/lo split
    # [32][128], the norms, the guard count, h_r [300][32]
    assert full - saved == 3 * 32 * 128 * 2 + 512 + 256 + 300 * 32 * 2
    assert L.lora_bwd_workspace_layout(300, 64, 128, 17, 1, 1, 0, 1, 1, 1, 7 | 16)[0] == 2 ** 64 - 1


def test_forward_with_kept_compute_copy_checks():
    """lyc_lora_linear_fwd_wc: W_c read in place (16-byte aligned, no overlap
    with y), W's dtype still in the policy, and a workspace without the W copy
    with every other region at the same offset."""
    lib = L.lib()
    a = dict(x=P, x_dt=2, w=V(1 << 28), w_dt=3, b=None, b_dt=0, d=P, d_dt=3, u=P, u_dt=3, r=4, scale=1.0,
             y=V(1 << 30), y_dt=3, M=4, N=64, K=64, ws=None, nws=0, s=None)
    call = lambda **kw: _refused(lib.lyc_lora_linear_fwd_wc(*[{**a, **kw}[k] for k in (
        "x", "x_dt", "w", "w_dt", "b", "b_dt", "d", "d_dt", "u", "u_dt", "r")], ctypes.c_double({**a, **kw}["scale"]),
        *[{**a, **kw}[k] for k in ("y", "y_dt", "M", "N", "K", "ws", "nws", "s")]))
    assert call(w=None) == L.ERR_INVALID_ARG
    assert call(w=V((1 << 28) + 8)) == L.ERR_UNSUPPORTED          # W_c rows are read 16 bytes at a time
    assert call(w=V((1 << 30) + 512)) == L.ERR_INVALID_ARG         # overlaps y
    assert call(y_dt=2) == L.ERR_DTYPE_MISMATCH                    # fp32 W keeps y fp32
    assert call() == L.ERR_WORKSPACE
    # fp32 W under bf16 compute: exactly the bf16 copy of W less; bf16 W: no difference
    full = L.lora_workspace_size(300, 520, 264, 64, 2, 3, 0, 3, 3)
    n = ctypes.c_size_t(0)
    assert lib.lyc_lora_linear_wc_workspace_size(300, 520, 264, 64, 2, 3, 0, 3, 3, ctypes.byref(n)) == L.OK
    assert full - n.value == -(-520 * 264 * 2 // 256) * 256   # (regions are 256-byte aligned)
    assert lib.lyc_lora_linear_wc_workspace_size(300, 520, 264, 64, 2, 2, 0, 2, 2, ctypes.byref(n)) == L.OK
    assert n.value == L.lora_workspace_size(300, 520, 264, 64, 2, 2, 0, 2, 2)


def test_prepared_affine_checks():
    """lyc_linear_prepare / lyc_linear_fwd_prepared: the arguments and errors of
    lyc_linear_fwd (prepare reads only W), and nothing done for empty shapes."""
    lib = L.lib()
    ws_need = L.linear_workspace_size(1024, 1024, 768, 1, 1, 1)
    assert ws_need > 0
    prep = lambda ok=False, **kw: _refused(lib.lyc_linear_prepare(
        *[{**dict(w=V(1 << 28), w_dt=1, x_dt=1, b_dt=1, M=1024, N=1024, K=768, ws=None, nws=0, s=None), **kw}[k]
          for k in ("w", "w_dt", "x_dt", "b_dt", "M", "N", "K", "ws", "nws", "s")]), ok)
    assert prep(w=None) == L.ERR_INVALID_ARG
    assert prep(w=V((1 << 28) + 8)) == L.ERR_UNSUPPORTED
    assert prep() == L.ERR_WORKSPACE
    assert prep(ws=V(1 << 29), nws=ws_need - 1) == L.ERR_WORKSPACE
    assert prep(ws=V((1 << 29) + 16), nws=ws_need) == L.ERR_WORKSPACE   # not 256-byte aligned
    assert prep(x_dt=1, w_dt=2) == L.ERR_MIXED_HALF
    assert prep(True, M=0) == L.OK and prep(True, K=0) == L.OK
    fwd = lambda **kw: _refused(lib.lyc_linear_fwd_prepared(*[{**dict(x=V(1 << 27), x_dt=1, w=V(1 << 28), w_dt=1,
                                                                        b=V(1 << 26), b_dt=1, y=V(1 << 30), y_dt=1,
                                                                        M=1024, N=1024, K=768, ws=None, nws=0,
                                                                        s=None), **kw}[k]
                                                             for k in ("x", "x_dt", "w", "w_dt", "b", "b_dt", "y",
                                                                       "y_dt", "M", "N", "K", "ws", "nws", "s")]))
    assert fwd(w=None) == L.ERR_INVALID_ARG
    assert fwd(y_dt=3) == L.ERR_DTYPE_MISMATCH
    assert fwd() == L.ERR_WORKSPACE
