"""Plain fp64 CPU oracle for the LoRA-bypass linear -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The GPU library never calls it and shares no
code with it.  The arithmetic lives in ``oracle.c`` (binary64, rounding only at
the declared boundaries); this module marshals numpy arrays to it and holds
the scoring rules (tolerance, ULP) that judge a result against it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

F16, BF16, F32 = 1, 2, 3
OK, MIXED_HALF, INVALID = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point this at another build of oracle.c (e.g. a deliberately
# broken copy, to show that the pins catch the mistake).
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB_OVERRIDE")
_lib = None


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.c with gcc (IEEE semantics: no fast-math, no contraction).
    With ``sanitize``: an AddressSanitizer + UndefinedBehaviorSanitizer build,
    liboracle_san.so, for the CPU tests (run with gcc's libasan preloaded and
    ORACLE_LIB_OVERRIDE pointing at it)."""
    lib = _LIB.replace(".so", "_san.so") if sanitize else _LIB
    if force or not os.path.exists(lib):
        tmp = lib + f".tmp{os.getpid()}"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math"] + (san if sanitize else []) + ["-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, lib)
    return lib


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build()
            L = ctypes.CDLL(_LIB)
        L.oracle_round.restype = ctypes.c_double
        L.oracle_round.argtypes = [ctypes.c_double, ctypes.c_int]
        L.oracle_widen.restype = ctypes.c_double
        L.oracle_widen.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64]
        L.oracle_store.restype = None
        L.oracle_store.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double]
        for nm, args in (("oracle_round_n", [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]),
                         ("oracle_widen_n", [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64]),
                         ("oracle_store_n", [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64])):
            getattr(L, nm).restype = None
            getattr(L, nm).argtypes = args
        L.oracle_resolve.restype = ctypes.c_int
        L.oracle_resolve.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        L.oracle_forward.restype = ctypes.c_int
        L.oracle_merge.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        L.oracle_forward.argtypes = [ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_int64, ctypes.c_double,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_backward.restype = ctypes.c_int
        L.oracle_backward.argtypes = [vp, ci, vp, ci, ci, vp, ci, vp, ci, i64, ctypes.c_double, vp, ci,
                                      i64, i64, i64, vp, i64, vp, vp, vp, vp, i64, vp, i64, vp, vp, vp, i64,
                                      vp, vp, vp, vp, vp, ci, ctypes.POINTER(ctypes.c_int)]
        L.oracle_dora_norms.restype = ctypes.c_int
        L.oracle_dora_norms.argtypes = [vp, ci, vp, ci, vp, ci, i64, ctypes.c_double, i64, i64, vp, i64, vp, vp, ci,
                                        ctypes.POINTER(ctypes.c_int)]
        L.oracle_dora_forward.restype = ctypes.c_int
        L.oracle_dora_forward.argtypes = [vp, ci, vp, ci, vp, ci, vp, ci, vp, ci, vp, ci, i64, ctypes.c_double, i64,
                                          i64, i64, vp, i64, vp, vp, vp, ci, ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_int)]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    """Host threads for the oracle in the test suite: the CPUs this process may
    run on, at most 16."""
    return max(1, min(16, host_cpus()[0]))


def host_cpus():
    """(usable, affinity, quota): the CPUs this process may run on
    (sched_getaffinity), the cgroup CPU quota when one is set (cpu.max, in
    CPUs, else None), and their minimum -- every host core the process can
    actually use, which is what the benchmark's oracle baseline runs on."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, p = f.read().split()[:2]
        if q != "max" and int(p) > 0:
            quota = max(1, int(int(q) // int(p)))
    except (OSError, ValueError):
        quota = None
    usable = aff if quota is None else max(1, min(aff, quota))
    return usable, aff, quota


def storage_np(dt: int):
    return np.float32 if dt == F32 else np.uint16


# ---- elementwise helpers ----------------------------------------------------

def round_to(v: float, dt: int) -> float:
    """RNE of a binary64 value to dtype dt, returned as binary64."""
    return lib().oracle_round(float(v), int(dt))


def round_array(v: np.ndarray, dt: int) -> np.ndarray:
    """Elementwise RNE of binary64 values to dtype dt (as binary64)."""
    a = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(a)
    lib().oracle_round_n(_ptr(a), _ptr(out), a.size, int(dt))
    return out


def widen(bits: np.ndarray, dt: int) -> np.ndarray:
    """Stored elements (uint16 bit patterns or float32) -> exact float64."""
    a = np.ascontiguousarray(bits, dtype=storage_np(dt))
    out = np.empty(a.shape, dtype=np.float64)
    lib().oracle_widen_n(_ptr(a), int(dt), _ptr(out), a.size)
    return out


def encode(values: Sequence[float], dt: int) -> np.ndarray:
    """Representable binary64 values -> storage (uint16 bits or float32)."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.zeros(v.shape, dtype=storage_np(dt))
    lib().oracle_store_n(_ptr(out), int(dt), _ptr(v), v.size)
    return out


def resolve(dtypes: Sequence[int]):
    """Dtype policy: returns (status, compute, output)."""
    arr = (ctypes.c_int * max(1, len(dtypes)))(*dtypes)
    c, o = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().oracle_resolve(arr, len(dtypes), ctypes.byref(c), ctypes.byref(o))
    return st, c.value, o.value


# ---- the forward ------------------------------------------------------------

class OracleError(RuntimeError):
    def __init__(self, status):
        super().__init__({MIXED_HALF: "fp16 mixed with bf16", INVALID: "invalid argument"}.get(status, status))
        self.status = status


def forward(x, x_dt, w, w_dt, b=None, b_dt=None, down=None, down_dt=None, up=None, up_dt=None,
            scale: float = 1.0, rows=None, nthreads: Optional[int] = None, lora: bool = True,
            want_y=True, want_ref=True, want_h=True):
    """Evaluate the forward (LoRA when ``lora`` else the plain affine contract).

    Arrays are storage arrays (uint16 bit patterns for 16-bit, float32 for
    fp32): x [M,K], w [N,K], b [N], down [r,K], up [N,r].  ``rows`` selects the
    output rows to evaluate (default: all).  Returns a dict with the resolved
    ``compute``/``output`` dtypes, ``y`` (storage of the output dtype),
    ``ref`` (float64 value before the final rounding) and ``h`` (float64 value
    of h after its rounding), each [len(rows), N] / [len(rows), r]."""
    x = np.ascontiguousarray(x, dtype=storage_np(x_dt))
    w = np.ascontiguousarray(w, dtype=storage_np(w_dt))
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    if b is not None:
        b = np.ascontiguousarray(b, dtype=storage_np(b_dt))
        assert b.shape == (N,)
    r = 0
    if lora:
        down = np.ascontiguousarray(down, dtype=storage_np(down_dt))
        up = np.ascontiguousarray(up, dtype=storage_np(up_dt))
        r = down.shape[0]
        assert down.shape == (r, K) and up.shape == (N, r)
    if rows is None:
        rows_arr = None
        nrows = M
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    if nthreads is None:
        nthreads = default_threads()
    st, c_dt, o_dt = resolve([x_dt, w_dt] + ([b_dt] if b is not None else []) +
                             ([down_dt, up_dt] if lora else []))
    if st != OK:
        raise OracleError(st)
    y = np.zeros((nrows, N), dtype=storage_np(o_dt)) if want_y else None
    ref = np.zeros((nrows, N), dtype=np.float64) if want_ref else None
    h = np.zeros((nrows, r), dtype=np.float64) if (want_h and lora) else None
    c_out, o_out = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().oracle_forward(int(lora), _ptr(x), x_dt, _ptr(w), w_dt, _ptr(b), b_dt or 0,
                              _ptr(down), down_dt or 0, _ptr(up), up_dt or 0, r, float(scale),
                              M, N, K, _ptr(rows_arr), nrows, _ptr(y), _ptr(ref), _ptr(h), int(nthreads),
                              ctypes.byref(c_out), ctypes.byref(o_out))
    if st != OK:
        raise OracleError(st)
    return {"compute": c_out.value, "output": o_out.value, "y": y, "ref": ref, "h": h}


def merge(w, w_dt, down, down_dt, up, up_dt, scale: float = 1.0, rows=None, nthreads: Optional[int] = None):
    """The LoRA merge W' = round_out(W + scale * up_c . down_c) for the rows of
    W in ``rows`` (default: all).  Storage arrays as in ``forward``: w [N,K],
    down [r,K], up [N,r].  Returns a dict with the resolved ``compute`` /
    ``output`` dtypes, ``y`` (storage of the output dtype, [len(rows), K]) and
    ``ref`` (float64 value before the rounding)."""
    w = np.ascontiguousarray(w, dtype=storage_np(w_dt))
    down = np.ascontiguousarray(down, dtype=storage_np(down_dt))
    up = np.ascontiguousarray(up, dtype=storage_np(up_dt))
    N, K = w.shape
    r = down.shape[0]
    assert down.shape == (r, K) and up.shape == (N, r)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = N if rows is None else rows_arr.size
    st, c_dt, o_dt = resolve([w_dt, down_dt, up_dt])
    if st != OK:
        raise OracleError(st)
    y = np.zeros((nrows, K), dtype=storage_np(o_dt))
    ref = np.zeros((nrows, K), dtype=np.float64)
    c_out, o_out = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().oracle_merge(_ptr(w), w_dt, _ptr(down), down_dt, _ptr(up), up_dt, r, float(scale), N, K,
                            _ptr(rows_arr), nrows, _ptr(y), _ptr(ref),
                            int(default_threads() if nthreads is None else nthreads),
                            ctypes.byref(c_out), ctypes.byref(o_out))
    if st != OK:
        raise OracleError(st)
    return {"compute": c_out.value, "output": o_out.value, "y": y, "ref": ref}


def backward(x, x_dt, w, w_dt, down, down_dt, up, up_dt, dy, dy_dt, scale: float = 1.0, b_dt: int = 0,
             dx_rows=None, js=None, dd_cols=None, du_rows=None, nthreads: Optional[int] = None):
    """The LoRA-bypass backward for a given dy: dx = round_x(dy_c.W_c + gh_r.down_c),
    dDown = round_down(gh_r^T.x_c), dUp = round_up(scale * dy_c^T.h_r), with
    gh_r = round_c(scale * dy_c.up_c) and h_r the forward's rounded h.

    Storage arrays: x [M,K], w [N,K], down [r,K], up [N,r], dy [M,N]; b_dt is
    the forward's bias dtype (0: none; it only enters the dtype policy).
    Index sets (default: all) select the rows of dx (tokens), the rank
    indices js, the columns of dDown (k) and the rows of dUp (n).  Returns a
    dict with ``compute``, ``dx`` / ``dx_ref`` [len(dx_rows), K], ``gh``
    [len(dx_rows), r] (the rounded gh of those rows, float64), ``d_down`` /
    ``dd_ref`` [len(js), len(dd_cols)] and ``d_up`` / ``du_ref``
    [len(du_rows), len(js)]; gradients in storage of their leaf's dtype;
    ``dx_rss`` / ``dd_rss`` / ``du_rss``: the root-sum-square of the terms of
    each output's final sum (for ``tolerance_sum``)."""
    x = np.ascontiguousarray(x, dtype=storage_np(x_dt))
    w = np.ascontiguousarray(w, dtype=storage_np(w_dt))
    down = np.ascontiguousarray(down, dtype=storage_np(down_dt))
    up = np.ascontiguousarray(up, dtype=storage_np(up_dt))
    dy = np.ascontiguousarray(dy, dtype=storage_np(dy_dt))
    M, K = x.shape
    N = w.shape[0]
    r = down.shape[0]
    assert w.shape == (N, K) and down.shape == (r, K) and up.shape == (N, r) and dy.shape == (M, N)

    def idx(v, n):
        return np.arange(n, dtype=np.int64) if v is None else np.ascontiguousarray(v, dtype=np.int64)

    dx_rows, js, dd_cols, du_rows = idx(dx_rows, M), idx(js, r), idx(dd_cols, K), idx(du_rows, N)
    dx = np.zeros((dx_rows.size, K), dtype=storage_np(x_dt))
    dx_ref = np.zeros((dx_rows.size, K))
    gh = np.zeros((dx_rows.size, r))
    d_down = np.zeros((js.size, dd_cols.size), dtype=storage_np(down_dt))
    dd_ref = np.zeros((js.size, dd_cols.size))
    d_up = np.zeros((du_rows.size, js.size), dtype=storage_np(up_dt))
    du_ref = np.zeros((du_rows.size, js.size))
    dx_rss, dd_rss, du_rss = np.zeros_like(dx_ref), np.zeros_like(dd_ref), np.zeros_like(du_ref)
    c_out = ctypes.c_int(0)
    st = lib().oracle_backward(_ptr(x), x_dt, _ptr(w), w_dt, int(b_dt or 0), _ptr(down), down_dt, _ptr(up), up_dt,
                               r, float(scale), _ptr(dy), dy_dt, M, N, K, _ptr(dx_rows), dx_rows.size, _ptr(dx),
                               _ptr(dx_ref), _ptr(gh), _ptr(js), js.size, _ptr(dd_cols), dd_cols.size, _ptr(d_down),
                               _ptr(dd_ref), _ptr(du_rows), du_rows.size, _ptr(d_up), _ptr(du_ref), _ptr(dx_rss),
                               _ptr(dd_rss), _ptr(du_rss), int(default_threads() if nthreads is None else nthreads),
                               ctypes.byref(c_out))
    if st != OK:
        raise OracleError(st)
    return {"compute": c_out.value, "dx": dx, "dx_ref": dx_ref, "gh": gh, "d_down": d_down, "dd_ref": dd_ref,
            "d_up": d_up, "du_ref": du_ref, "dx_rss": dx_rss, "dd_rss": dd_rss, "du_rss": du_rss}


def dora_norms(w, w_dt, down, down_dt, up, up_dt, scale: float = 1.0, rows=None, nthreads: Optional[int] = None):
    """DoRA row norms RN_fp32(||W + scale * up_c.down_c||_2) for the rows of W
    in ``rows`` (default all).  Returns (norms float32, exact float64, compute)."""
    w = np.ascontiguousarray(w, dtype=storage_np(w_dt))
    down = np.ascontiguousarray(down, dtype=storage_np(down_dt))
    up = np.ascontiguousarray(up, dtype=storage_np(up_dt))
    N, K = w.shape
    r = down.shape[0]
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = N if rows is None else rows_arr.size
    norms = np.zeros(nrows, dtype=np.float32)
    exact = np.zeros(nrows)
    c_out = ctypes.c_int(0)
    st = lib().oracle_dora_norms(_ptr(w), w_dt, _ptr(down), down_dt, _ptr(up), up_dt, r, float(scale), N, K,
                                 _ptr(rows_arr), nrows, _ptr(norms), _ptr(exact),
                                 int(default_threads() if nthreads is None else nthreads), ctypes.byref(c_out))
    if st != OK:
        raise OracleError(st)
    return norms, exact, c_out.value


def dora_forward(x, x_dt, w, w_dt, b, b_dt, down, down_dt, up, up_dt, mag, m_dt, scale: float = 1.0, rows=None,
                 nthreads: Optional[int] = None):
    """The DoRA forward y = round_out((m/norm) * (x_c.W_c^T + scale h_r.up_c^T) + b)
    with the fp32 row norms computed here.  Returns a dict like ``forward`` plus
    ``norms`` (float32 [N])."""
    x = np.ascontiguousarray(x, dtype=storage_np(x_dt))
    w = np.ascontiguousarray(w, dtype=storage_np(w_dt))
    down = np.ascontiguousarray(down, dtype=storage_np(down_dt))
    up = np.ascontiguousarray(up, dtype=storage_np(up_dt))
    mag = np.ascontiguousarray(mag, dtype=storage_np(m_dt))
    if b is not None:
        b = np.ascontiguousarray(b, dtype=storage_np(b_dt))
    M, K = x.shape
    N = w.shape[0]
    r = down.shape[0]
    assert mag.shape == (N,) and up.shape == (N, r) and down.shape == (r, K)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = M if rows is None else rows_arr.size
    dts = [x_dt, w_dt] + ([b_dt] if b is not None else []) + [down_dt, up_dt, m_dt]
    st, c_dt, o_dt = resolve(dts)
    if st != OK:
        raise OracleError(st)
    y = np.zeros((nrows, N), dtype=storage_np(o_dt))
    ref = np.zeros((nrows, N))
    norms = np.zeros(N, dtype=np.float32)
    c_out, o_out = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().oracle_dora_forward(_ptr(x), x_dt, _ptr(w), w_dt, _ptr(b), b_dt or 0, _ptr(down), down_dt, _ptr(up),
                                   up_dt, _ptr(mag), m_dt, r, float(scale), M, N, K, _ptr(rows_arr), nrows, _ptr(y),
                                   _ptr(ref), _ptr(norms), int(default_threads() if nthreads is None else nthreads),
                                   ctypes.byref(c_out), ctypes.byref(o_out))
    if st != OK:
        raise OracleError(st)
    return {"compute": c_out.value, "output": o_out.value, "y": y, "ref": ref, "norms": norms}


# ---- scoring ----------------------------------------------------------------

# Per-element tolerance abs(actual - reference) <= atol + rtol*abs(reference).
# fp16 bound from the Luminal FP16 page ("Validation and Experimental Design");
# the bf16 bound is the fp16 one widened by bf16's three fewer significand bits
# (x8).  An fp32 output produced from 16-bit compute uses the 16-bit bound.
TOL = {F16: (2e-4, 2e-3), BF16: (2e-3, 1.6e-2)}

# significand bits and minimum normal exponent of each working dtype
_P = {F16: (11, -14), BF16: (8, -126), F32: (24, -126)}


def tolerance(ref: np.ndarray, compute: int, K: int, r: int) -> np.ndarray:
    """Per-element bound for |gpu - ref|.  16-bit compute: the bound above.
    fp32 compute (no bound on the pages): 8 * 2^-24 * sqrt(K + r) * (1 + |ref|),
    a multiple of the expected fp32 accumulation error of a (K + r)-term sum."""
    a = np.abs(ref)
    if compute in TOL:
        atol, rtol = TOL[compute]
        return atol + rtol * a
    return 8.0 * 2.0 ** -24 * np.sqrt(max(K + r, 1)) * (1.0 + a)


def tolerance_sum(ref: np.ndarray, rss: np.ndarray, compute: int, L: int) -> np.ndarray:
    """Per-element bound for |gpu - ref| of a result summed over L terms whose
    root-sum-square is rss (the gradients).  The fp32 accumulation a GPU does
    errs by about 2^-24 * sqrt(L) times the size of its partial sums, which
    for terms of random sign is rss, not |ref|: 8 * 2^-24 * sqrt(L) * rss.
    16-bit compute: the forward's bound plus that term; fp32 compute:
    8 * 2^-24 * sqrt(L) * (|ref| + rss) (the forward's (1 + |ref|) with the
    terms' own scale in place of the 1)."""
    a = np.abs(ref)
    acc = 8.0 * 2.0 ** -24 * np.sqrt(max(L, 1)) * rss
    if compute in TOL:
        atol, rtol = TOL[compute]
        return atol + rtol * a + acc
    return 8.0 * 2.0 ** -24 * np.sqrt(max(L, 1)) * a + acc


def ulp_of(v: float, dt: int) -> float:
    """Spacing of dtype dt at magnitude v: 2^(max(floor(log2 v), emin) - p + 1)."""
    p, emin = _P[dt]
    if not np.isfinite(v) or v <= 0:
        return 2.0 ** (emin - p + 1)
    e = max(int(np.floor(np.log2(v))), emin)
    return 2.0 ** (e - p + 1)


def ulp_report(actual: np.ndarray, ref64: np.ndarray, working: int):
    """ULP of the working dtype against the fp64 reference, scored relative to
    the reference's RMS (LyCORIS "Precision" page, "Measured accuracy").
    Returns (max, rms)."""
    ref64 = np.asarray(ref64, dtype=np.float64)
    act = np.asarray(actual, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref64 ** 2))) if ref64.size else 0.0
    u = ulp_of(rms, working)
    e = np.abs(act - ref64) / u
    if e.size == 0:
        return 0.0, 0.0
    return float(np.max(e)), float(np.sqrt(np.mean(e ** 2)))


def as_float64(y: np.ndarray, dt: int) -> np.ndarray:
    """Storage array -> float64 values (vectorised exact widening)."""
    if dt == F32:
        return np.asarray(y, dtype=np.float32).astype(np.float64)
    if dt == F16:
        return np.asarray(y, dtype=np.uint16).view(np.float16).astype(np.float64)
    u = np.asarray(y, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
