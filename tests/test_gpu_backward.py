"""GPU parity of the LoRA-bypass backward against the fp64 oracle, through the
C ABI, element by element.

Bar: gh_r (the rounded gradient at h) identical, bit for bit, to the oracle's
under 16-bit compute; dx, dDown and dUp within ``oracle.tolerance_sum``: the
forward's per-element bound of the compute dtype (fp16 2e-4 + 2e-3|ref|, bf16
2e-3 + 1.6e-2|ref|) plus the fp32 accumulation term 8 * 2^-24 * sqrt(L) * rss,
with L the contraction length (N + r for dx, M for dDown and dUp) and rss the
root-sum-square of the sum's terms; fp32 compute: 8 * 2^-24 * sqrt(L) *
(|ref| + rss).  Full outputs at sizes
spanning several tiles with ragged edges; sampled rows, columns and rank
indices at the full workload shapes.
"""
import numpy as np
import pytest
import torch

import lora_bypass_linear_amd as L
import oracle
import workloads as WL
from tests.gpu_cases import say, sample_rows

pytestmark = pytest.mark.gpu

BASE = WL.WORKLOADS
_T = {L.F16: torch.float16, L.BF16: torch.bfloat16, L.F32: torch.float32}


def _inputs(wl, dy_dt=None):
    inp = WL.generate(wl)
    dts = [WL.dtype_code(inp[k]) for k in ("x", "w", "down", "up")] + ([WL.dtype_code(inp["b"])] if "b" in inp else [])
    _, o_dt = L.resolve_dtypes(dts)
    inp["dy"] = WL.generate_dy(wl, o_dt if dy_dt is None else dy_dt)
    return inp


def _gpu(inp, wl, scale=None, want=(True, True, True)):
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inp.items()}
    s = wl.scale if scale is None else scale
    say("backward", wl.name, f"M={wl.M} N={wl.N} K={wl.K} r={wl.r} scale={s} want={want}")
    b_dtype = inp["b"].dtype if "b" in inp else None
    (dx, dd, du), ws = L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], s, d["dy"], bias_dtype=b_dtype,
                                              want_dx=want[0], want_ddown=want[1], want_dup=want[2],
                                              return_workspace=True)
    torch.cuda.synchronize()
    codes = [WL.dtype_code(inp[k]) for k in ("x", "w")] + [WL.dtype_code(inp["b"]) if "b" in inp else 0] + \
            [WL.dtype_code(inp[k]) for k in ("down", "up", "dy")]
    wmask = (1 if want[0] else 0) | (2 if want[1] else 0) | (4 if want[2] else 0)
    ho, go, ld, fo = L.lora_bwd_workspace_layout(wl.M, wl.N, wl.K, wl.r, *codes, want=wmask)
    c_dt, _ = L.resolve_dtypes([c for c in codes if c])
    gh = None
    if ws is not None and go != 2 ** 64 - 1 and wl.M > 0 and wl.r > 0:
        es = 4 if c_dt == L.F32 else 2
        raw = ws[go: go + wl.M * ld * es].cpu()
        if c_dt == L.F32:
            gh = raw.view(torch.float32).numpy().reshape(wl.M, ld).astype(np.float64)[:, :wl.r]
        else:
            gh = oracle.as_float64(raw.view(torch.int16).numpy().view(np.uint16).reshape(wl.M, ld), c_dt)[:, :wl.r]
    out = lambda t: None if t is None else t.cpu()
    return out(dx), out(dd), out(du), gh


def _oracle(inp, wl, scale=None, **idx):
    b = {k: WL.raw_bits(v) for k, v in inp.items()}
    dt = {k: WL.dtype_code(v) for k, v in inp.items()}
    return oracle.backward(b["x"], dt["x"], b["w"], dt["w"], b["down"], dt["down"], b["up"], dt["up"], b["dy"],
                           dt["dy"], scale=(wl.scale if scale is None else scale), b_dt=dt.get("b", 0), **idx)


def _score(name, gpu, want, ref, rss, dt, c_dt, length):
    """Element-wise tolerance check of one gradient (storage arrays)."""
    g = oracle.as_float64(WL.raw_bits(gpu) if isinstance(gpu, torch.Tensor) else gpu, dt)
    w = oracle.as_float64(want, dt)
    tol = oracle.tolerance_sum(w, rss, c_dt, length)
    with np.errstate(invalid="ignore"):
        ok = (g == w) | (np.abs(g - w) <= tol)
    bad = np.argwhere(~ok)
    umax, urms = oracle.ulp_report(g[np.isfinite(g)], ref[np.isfinite(g)], c_dt) if g.size else (0.0, 0.0)
    print(name, "n", g.size, "fail", bad.shape[0], "ulp max/rms", round(umax, 3), round(urms, 3))
    assert bad.shape[0] == 0, (name, bad[:5].tolist(), g[tuple(bad[0])], w[tuple(bad[0])])


def _check(wl, inp=None, scale=None, want=(True, True, True), dx_rows=None, js=None, dd_cols=None, du_rows=None):
    inp = inp if inp is not None else _inputs(wl)
    dx, dd, du, gh = _gpu(inp, wl, scale, want)
    res = _oracle(inp, wl, scale, dx_rows=dx_rows, js=js, dd_cols=dd_cols, du_rows=du_rows)
    c_dt = res["compute"]
    dt = {k: WL.dtype_code(v) for k, v in inp.items()}
    rows = np.arange(wl.M) if dx_rows is None else np.asarray(dx_rows)
    jj = np.arange(wl.r) if js is None else np.asarray(js)
    kk = np.arange(wl.K) if dd_cols is None else np.asarray(dd_cols)
    nn = np.arange(wl.N) if du_rows is None else np.asarray(du_rows)
    if want[0]:
        _score("dx", WL.raw_bits(dx)[rows], res["dx"], res["dx_ref"], res["dx_rss"], dt["x"], c_dt, wl.N + wl.r)
    if want[1] and wl.r > 0:
        _score("dDown", WL.raw_bits(dd)[np.ix_(jj, kk)], res["d_down"], res["dd_ref"], res["dd_rss"], dt["down"], c_dt,
               wl.M)
    if want[2] and wl.r > 0:
        _score("dUp", WL.raw_bits(du)[np.ix_(nn, jj)], res["d_up"], res["du_ref"], res["du_rss"], dt["up"], c_dt, wl.M)
    if gh is not None and (want[0] or want[1]) and c_dt != L.F32 and wl.M > 0:
        mism = np.argwhere(gh[rows] != res["gh"])
        assert mism.size == 0, f"gh_r differs from the oracle at {mism[:5].tolist()}"
    return res


# ---- the LoRA workloads at oracle-friendly sizes (several tiles, ragged tails) ------

SMALL = {
    "lora_f16_4096x3072x3072_r16": dict(M=300, K=392, N=336),
    "lora_bf16x_f32w_8192x4096x4096_r64": dict(M=257, K=264, N=200),
    "lora_bf16_16384x8192x8192_r128": dict(M=270, K=520, N=304),
}
SMALL.update({n: dict(M=130, K=136, N=264) for n in WL.SWEEP
              if (BASE[n].x_dt, BASE[n].w_dt) not in ((1, 2), (2, 1))})


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_output(name):
    _check(BASE[name].resized(**SMALL[name]))


EDGE = [
    ("rank0", "lora_f16_4096x3072x3072_r16", dict(M=65, N=72, K=64, r=0), None),
    ("rank1", "lora_f16_4096x3072x3072_r16", dict(M=65, N=72, K=64, r=1), None),
    ("rank17", "lora_bf16_16384x8192x8192_r128", dict(M=100, N=96, K=136, r=17), None),
    ("rank256", "lora_f16_4096x3072x3072_r16", dict(M=70, N=64, K=128, r=256), None),
    ("m_ragged", "lora_f16_4096x3072x3072_r16", dict(M=13, N=40, K=48, r=16), None),
    ("m_one", "lora_bf16_16384x8192x8192_r128", dict(M=1, N=8, K=8, r=3), None),
    ("scale_neg", "lora_bf16_16384x8192x8192_r128", dict(M=64, N=96, K=256, r=32), -0.75),
    ("scale_zero", "lora_f16_4096x3072x3072_r16", dict(M=64, N=64, K=64, r=16), 0.0),
    ("fp32_all", "sweep_xf32_wf32_2048x1280x5120_r32", dict(M=100, N=136, K=72, r=32), None),
    # token contractions split four ways over 1000 tokens (the last split ragged)
    ("tok_split", "lora_bf16_16384x8192x8192_r128", dict(M=1000, N=72, K=136, r=17), None),
    # the largest token count the backward takes (2^20): token sums of 16384 K steps
    ("m_max", "lora_bf16_16384x8192x8192_r128", dict(M=1 << 20, N=16, K=16, r=8), None),
]


@pytest.mark.parametrize("tag,name,dims,scale", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(tag, name, dims, scale):
    _check(BASE[name].resized(**dims), scale=scale)


@pytest.mark.parametrize("want", [(True, False, False), (False, True, False), (False, False, True), (False, True, True)])
def test_partial_requests(want):
    wl = BASE["lora_bf16_16384x8192x8192_r128"].resized(M=96, N=80, K=72, r=24)
    _check(wl, want=want)


def test_fp32_dy_under_16bit_compute():
    wl = BASE["lora_f16_4096x3072x3072_r16"].resized(M=70, N=64, K=96)
    _check(wl, inp=_inputs(wl, dy_dt=L.F32))


def test_no_tokens():
    wl = BASE["lora_f16_4096x3072x3072_r16"].resized(M=0, N=64, K=96, r=8)
    dx, dd, du, _ = _gpu(_inputs(wl), wl)
    assert dx.shape == (0, 96) and not dd.float().abs().sum() and not du.float().abs().sum()


def test_mixed_halves_refused():
    wl = BASE["lora_f16_4096x3072x3072_r16"].resized(M=16, N=16, K=16)
    inp = _inputs(wl, dy_dt=L.BF16)
    with pytest.raises(L.MixedHalfError):
        _gpu(inp, wl)


@pytest.mark.parametrize("dims", [dict(M=200, N=136, K=264), dict(M=1000, N=72, K=136, r=17)],
                         ids=["one_split", "token_sums_split"])
def test_deterministic(dims):
    """Bit-identical gradients on repeated calls, also where the token sums
    are split over K (their partial sums are added in a fixed order)."""
    wl = BASE["lora_bf16_16384x8192x8192_r128"].resized(**dims)
    inp = _inputs(wl)
    a, b = _gpu(inp, wl), _gpu(inp, wl)
    for u, v in zip(a[:3], b[:3]):
        assert torch.equal(u, v)


# ---- the full workload shapes, sampled ----------------------------------------------

FULL = ["lora_f16_4096x3072x3072_r16", "lora_bf16x_f32w_8192x4096x4096_r64", "lora_bf16_16384x8192x8192_r128"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    wl = BASE[name]
    rng = np.random.default_rng(wl.seed)
    _check(wl, dx_rows=sample_rows(wl.M, 16, seed=wl.seed), js=np.sort(rng.choice(wl.r, 4, replace=False)),
           dd_cols=sample_rows(wl.K, 24, seed=wl.seed + 1), du_rows=sample_rows(wl.N, 24, seed=wl.seed + 2))


@pytest.mark.parametrize("name,dims", [
    ("lora_f16_4096x3072x3072_r16", dict(M=300, N=264, K=136)),
    ("lora_bf16_16384x8192x8192_r128", dict(M=130, N=520, K=264)),
    ("lora_bf16x_f32w_8192x4096x4096_r64", dict(M=200, N=136, K=72)),   # fp32 W: w_t is W rounded to bf16
    ("lora_f16_4096x3072x3072_r16", dict(M=16)),                         # dx splits K at this size
])
def test_caller_kept_wt_gives_identical_gradients(name, dims):
    """lyc_lora_linear_bwd_wt (W_c^T passed in, no per-call copy) against
    lyc_lora_linear_bwd: every gradient bit for bit."""
    wl = BASE[name].resized(**dims)
    inp = _inputs(wl)
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inp.items()}
    b_dtype = inp["b"].dtype if "b" in inp else None
    codes = [WL.dtype_code(inp[k]) for k in ("x", "w", "down", "up", "dy")] + \
            ([WL.dtype_code(inp["b"])] if "b" in inp else [])
    c_dt, _ = L.resolve_dtypes(codes)
    w_t = d["w"].to(_T[c_dt]).t().contiguous()
    say("backward w_t", wl.name, dims)
    ref = L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], wl.scale, d["dy"], bias_dtype=b_dtype)
    got = L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], wl.scale, d["dy"], bias_dtype=b_dtype, w_t=w_t)
    dxo = L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], wl.scale, d["dy"], bias_dtype=b_dtype, w_t=w_t,
                                 want_ddown=False, want_dup=False)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    assert torch.equal(ref[0], dxo[0]) and dxo[1] is None and dxo[2] is None


@pytest.mark.parametrize("name,dims", [
    ("lora_f16_4096x3072x3072_r16", dict(M=300, N=264, K=136)),
    ("lora_bf16_16384x8192x8192_r128", dict(M=1030, N=520, K=264)),     # bias; dUp on 128x128 tiles, K split
    ("lora_bf16x_f32w_8192x4096x4096_r64", dict(M=200, N=136, K=72)),
    ("sweep_xf32_wf32_2048x1280x5120_r32", dict(M=130, N=96, K=64)),     # fp32 compute: dUp reads a copy of h_r^T
])
def test_saved_h_gives_identical_gradients(name, dims):
    """lyc_lora_linear_bwd_saved with the h_r the forward left in its
    workspace (no h pass), alone and with a caller-kept W_c^T, against
    lyc_lora_linear_bwd: every gradient bit for bit."""
    wl = BASE[name].resized(**dims)
    inp = _inputs(wl)
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inp.items()}
    b_dtype = inp["b"].dtype if "b" in inp else None
    codes = [WL.dtype_code(inp[k]) for k in ("x", "w", "down", "up", "dy")] + \
            ([WL.dtype_code(inp["b"])] if "b" in inp else [])
    c_dt, _ = L.resolve_dtypes(codes)
    say("backward saved h", wl.name, dims)
    _, ws = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), return_workspace=True)
    h = L.lora_saved_h(ws, d["x"], d["w"], d["down"], d["up"], d.get("b"))
    ref = L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], wl.scale, d["dy"], bias_dtype=b_dtype)
    got = L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], wl.scale, d["dy"], bias_dtype=b_dtype, h=h)
    w_t = d["w"].to(_T[c_dt]).t().contiguous()
    both = L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], wl.scale, d["dy"], bias_dtype=b_dtype, h=h,
                                  w_t=w_t)
    duo = L.lora_linear_backward(d["x"], d["w"], d["down"], d["up"], wl.scale, d["dy"], bias_dtype=b_dtype, h=h,
                                 want_dx=False, want_ddown=False)
    torch.cuda.synchronize()
    for a, b, c in zip(ref, got, both):
        assert torch.equal(a, b) and torch.equal(a, c)
    assert duo[0] is None and duo[1] is None and torch.equal(ref[2], duo[2])
