"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs, element by element.

Bar: every element within abs(gpu - ref) <= atol + rtol*|ref| (fp16: 2e-4 +
2e-3|ref|, Luminal FP16 page; bf16: 2e-3 + 1.6e-2|ref|; fp32 output from
16-bit compute: the 16-bit bound; fp32 compute: 8*2^-24*sqrt(K+r)*(1+|ref|)),
and the rounded h identical, bit for bit, to the oracle's for 16-bit compute.
"""
import numpy as np
import pytest
import torch

import lora_bypass_linear_amd as L
import oracle
import workloads as WL
from tests import exact
from tests.gpu_cases import gpu_forward, oracle_forward, say, sample_rows, score

pytestmark = pytest.mark.gpu

BASE = WL.WORKLOADS


def _check(wl, inputs=None, rows=None, scale=None, h_exact=True):
    inputs = inputs if inputs is not None else WL.generate(wl)
    y, h, flagged = gpu_forward(inputs, wl, scale=scale)
    res = oracle_forward(inputs, wl, rows=rows, scale=scale)
    s = score(y, res, rows, wl.K, wl.r)
    print(wl.name, {k: v for k, v in s.items() if k != "first_bad"}, "flagged", flagged)
    assert s["fail"] == 0, s
    if wl.kind == "lora" and wl.r > 0:
        hr = h if rows is None else h[np.asarray(rows)]
        if s["compute"] != L.F32 and h_exact:
            mism = np.argwhere(hr != res["h"])
            assert mism.size == 0, f"h_r differs from the oracle at {mism[:5].tolist()}"
    return s


# ---- the hand-built boundary fixtures, through the library ----------------------

FIXTURES = exact.load_fixtures()


@pytest.mark.parametrize("fx", FIXTURES, ids=[f["name"] for f in FIXTURES])
def test_fixture_on_gpu(fx):
    a = exact.fixture_arrays(fx)
    dt = a["dt"]
    tdt = {1: torch.float16, 2: torch.bfloat16}[dt]
    dev = torch.device("cuda:0")

    def t(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(tdt).to(dev)

    say("fixture", fx["name"])
    b = t(a["b"]) if a["b"] is not None else None
    if fx["kind"] == "lora":
        y = L.lora_linear(t(a["x"]), t(a["w"]), t(a["down"]), t(a["up"]), a["scale"], b)
    else:
        y = L.linear(t(a["x"]), t(a["w"]), b)
    torch.cuda.synchronize()
    assert float(y.float().item()) == float(fx["expect"]), (fx["name"], float(y.float().item()))


# ---- every workload at oracle-friendly sizes (all tiles, ragged tails) -----------

SMALL = {
    "affine_f16_1024x768x1024": dict(M=300, K=264, N=333),
    "lora_f16_4096x3072x3072_r16": dict(M=300, K=392, N=333),
    "lora_bf16x_f32w_8192x4096x4096_r64": dict(M=257, K=264, N=200),
    "lora_bf16_16384x8192x8192_r128": dict(M=270, K=520, N=300),
}
SMALL.update({n: dict(M=130, K=136, N=260) for n in WL.SWEEP})


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_output(name):
    wl = BASE[name].resized(**SMALL[name])
    if wl.kind == "lora" and ((wl.x_dt, wl.w_dt) in ((1, 2), (2, 1))):
        inputs = WL.generate(wl)
        with pytest.raises(L.MixedHalfError):
            gpu_forward(inputs, wl)
        return
    _check(wl)


# shapes chosen so that each output-tile configuration runs, with ragged M, N and K
TILE_SHAPES = [(300, 333, 264), (1000, 2500, 392), (2600, 3100, 264), (3100, 4000, 136)]


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
@pytest.mark.parametrize("name", ["lora_f16_4096x3072x3072_r16", "lora_bf16_16384x8192x8192_r128",
                                  "affine_f16_1024x768x1024"])
def test_tiles_sampled_rows(name, M, N, K):
    wl = BASE[name].resized(M=M, N=N, K=K)
    _check(wl, rows=sample_rows(M, 24, seed=M))


# every h-pass work split: large M selects the wide-wave splits for ranks 64 and 128
@pytest.mark.parametrize("r", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("M", [8192, 16384])
def test_h_pass_splits_large_m(M, r):
    wl = BASE["lora_bf16_16384x8192x8192_r128"].resized(M=M, N=72, K=200, r=r)
    _check(wl, rows=sample_rows(M, 24, seed=r))


# decode-sized M: the shapes of the bench's small-M timings, every output row
# (the LoRA GEMM splits K over several workgroups there)
@pytest.mark.parametrize("M", [16, 128])
@pytest.mark.parametrize("name", ["affine_f16_1024x768x1024", "lora_f16_4096x3072x3072_r16"])
def test_small_m_full_output(name, M):
    _check(BASE[name].resized(M=M))


# K-split GEMM with a bias (bf16), with fp32 weights and fp32 output, and a ragged N
@pytest.mark.parametrize("name,dims", [("lora_bf16_16384x8192x8192_r128", dict(M=16, N=2048, K=1024)),
                                       ("lora_bf16x_f32w_8192x4096x4096_r64", dict(M=16, N=4096, K=1024)),
                                       ("lora_f16_4096x3072x3072_r16", dict(M=5, N=1003, K=1040))])
def test_k_split_gemm(name, dims):
    assert L.lora_workspace_size(dims["M"], dims["N"], dims["K"], 16, 1, 1, 0, 1, 1) > 0
    _check(BASE[name].resized(**dims))


def test_every_tile_configuration_is_covered():
    tiles = {L.gemm_tile(M, N, L.F16) for M, N, _ in TILE_SHAPES}
    assert tiles == {(64, 64), (128, 128), (192, 256), (256, 256)}
    assert {L.gemm_tile(M, N, L.F16) for M, N, _ in TILE_SHAPES_ROWS} == tiles


# the same tiles with y's rows a multiple of 16 bytes: the epilogue that stores
# whole rows through LDS (16-bit y in one pass; fp32 y of the 256-row tiles in
# two), with ragged M and K
TILE_SHAPES_ROWS = [(300, 336, 264), (1000, 2504, 392), (2600, 3104, 264), (3100, 4000, 136)]


@pytest.mark.parametrize("M,N,K", TILE_SHAPES_ROWS)
@pytest.mark.parametrize("name", ["lora_f16_4096x3072x3072_r16", "lora_bf16_16384x8192x8192_r128",
                                  "lora_bf16x_f32w_8192x4096x4096_r64"])
def test_tiles_whole_row_stores(name, M, N, K):
    wl = BASE[name].resized(M=M, N=N, K=K)
    _check(wl, rows=sample_rows(M, 24, seed=N))


def test_fp32_compute_tiles():
    wl = BASE["sweep_xf32_wf32_2048x1280x5120_r32"].resized(M=1000, N=2500, K=136)
    assert L.gemm_tile(1000, 2500, L.F32) == (128, 128)
    _check(wl, rows=sample_rows(1000, 24))


# ---- edge cases ---------------------------------------------------------------------

EDGE = [
    ("one_by_one", "lora_f16_4096x3072x3072_r16", dict(M=1, N=1, K=8, r=1), None),
    ("k_zero", "lora_bf16_16384x8192x8192_r128", dict(M=5, N=7, K=0, r=3), None),
    ("rank_one", "lora_f16_4096x3072x3072_r16", dict(M=65, N=70, K=72, r=1), None),
    ("rank_17", "lora_f16_4096x3072x3072_r16", dict(M=65, N=70, K=72, r=17), None),
    ("rank_200", "lora_bf16_16384x8192x8192_r128", dict(M=100, N=90, K=264, r=200), None),
    ("rank_256", "lora_f16_4096x3072x3072_r16", dict(M=70, N=64, K=128, r=256), None),
    ("odd_n", "lora_f16_4096x3072x3072_r16", dict(M=67, N=131, K=64, r=16), None),
    ("scale_3", "lora_f16_4096x3072x3072_r16", dict(M=64, N=64, K=256, r=16), 3.0),
    ("scale_neg", "lora_bf16_16384x8192x8192_r128", dict(M=64, N=96, K=256, r=32), -0.75),
    ("affine_k8", "affine_f16_1024x768x1024", dict(M=3, N=5, K=8), None),
    ("affine_odd_n", "affine_f16_1024x768x1024", dict(M=70, N=99, K=64), None),
    # the largest K the library takes (2^20): the longest accumulation chains and row offsets
    ("k_max_f16", "lora_f16_4096x3072x3072_r16", dict(M=20, N=40, K=1 << 20, r=16), None),
    ("k_max_bf16", "lora_bf16_16384x8192x8192_r128", dict(M=17, N=24, K=1 << 20, r=8), None),
    ("affine_k_max", "affine_f16_1024x768x1024", dict(M=9, N=24, K=1 << 20), None),
]


@pytest.mark.parametrize("tag,name,dims,scale", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(tag, name, dims, scale):
    wl = BASE[name].resized(**dims)
    _check(wl, scale=scale)


def _shifted(t):
    """t copied one element into a fresh buffer: element-aligned, not 16-byte aligned."""
    buf = torch.zeros(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


def test_unaligned_factors():
    """down and up one element into their buffers: the prepared copies are used
    instead of reading them as stored, with the same results."""
    wl = BASE["lora_f16_4096x3072x3072_r16"].resized(M=130, N=136, K=264)
    inputs = WL.generate(wl)
    d = {k: v.to(torch.device("cuda:0")) for k, v in inputs.items()}
    say("unaligned factors", wl.name)
    y_al, ws = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), return_workspace=True)
    args = (wl.M, wl.N, wl.K, wl.r, L.dtype_code(d["x"]), L.dtype_code(d["w"]),
            L.dtype_code(d["b"]) if "b" in d else 0, L.dtype_code(d["down"]), L.dtype_code(d["up"]))
    _, _, fo, ns = L.lora_workspace_layout(*args)
    # aligned, rank 16: the h pass splits down itself and counts per workgroup;
    # unaligned: down is prepared, one counter, and every other slot cleared
    assert ns > 1
    torch.cuda.synchronize()
    flagged_al = int(ws[fo: fo + 4 * ns].cpu().view(torch.int32).sum().item())
    ws.fill_(0xFF)
    y_un = L.lora_linear(d["x"], d["w"], _shifted(d["down"]), _shifted(d["up"]), wl.scale, d.get("b"), workspace=ws)
    torch.cuda.synchronize()
    flagged_un = int(ws[fo: fo + 4 * ns].cpu().view(torch.int32).sum().item())
    s = score(y_un.cpu(), oracle_forward(inputs, wl), None, wl.K, wl.r)
    assert s["fail"] == 0, s
    assert torch.equal(y_al.cpu(), y_un.cpu())
    assert flagged_al == flagged_un, (flagged_al, flagged_un)


def test_rank_zero_is_single_rounding():
    wl = BASE["lora_f16_4096x3072x3072_r16"].resized(M=40, N=48, K=64, r=0)
    _check(wl)


def test_empty_tokens():
    dev = torch.device("cuda:0")
    x = torch.empty((0, 64), dtype=torch.float16, device=dev)
    w = torch.randn(32, 64, device=dev).half()
    d = torch.randn(4, 64, device=dev).half()
    u = torch.randn(32, 4, device=dev).half()
    say("empty tokens")
    y = L.lora_linear(x, w, d, u, 1.0)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)


@pytest.mark.parametrize("M", [32, 160])   # the few-row GEMM (M <= 128) and the tiled one
def test_overflow_to_inf_matches(M):
    """Outputs beyond fp16's range: +-inf on both sides, sign for sign.  These
    inputs are scaled far past the pages' workloads, and some finite outputs
    cancel from sum|terms| ~ 5e5 to below 1, where any fp32 accumulation order
    errs by far more than the per-element bound of the pages' validation
    (Luminal FP16 page, "Validation and Experimental Design", which assumes
    their workloads).  Finite outputs are therefore held to that bound plus
    the fp32 accumulation term of oracle.tolerance_sum over the K + r products
    (the bound the gradients use), computed from the exact terms."""
    wl = BASE["lora_f16_4096x3072x3072_r16"].resized(M=M, N=40, K=64, r=16)
    inputs = WL.generate(wl)
    inputs["x"] = (inputs["x"].float() * 3000).clamp(-60000, 60000).half()
    inputs["w"] = (inputs["w"].float() * 200).half()                          # many outputs beyond fp16 range
    res = oracle_forward(inputs, wl)
    ref = oracle.as_float64(res["y"], oracle.F16)
    assert np.isinf(ref).mean() > 0.2
    y, _, _ = gpu_forward(inputs, wl)
    g = oracle.as_float64(WL.raw_bits(y), oracle.F16)
    inf = np.isinf(ref)
    # at the overflow threshold (max + half an ulp) the fp32 sum may land either side
    near = np.abs(np.abs(res["ref"]) - (65504.0 + 16.0)) <= oracle.tolerance(np.full(ref.shape, 65520.0), oracle.F16,
                                                                           wl.K, wl.r)
    agree = (np.isinf(g) == inf) | near
    assert agree.all(), np.argwhere(~agree)[:5]
    assert (np.sign(g[inf & np.isinf(g)]) == np.sign(ref[inf & np.isinf(g)])).all()
    # finite outputs: the pages' bound plus the fp32 accumulation term over the terms
    x, w = inputs["x"].double().numpy(), inputs["w"].double().numpy()
    d, u = inputs["down"].double().numpy(), inputs["up"].double().numpy()
    h = torch.from_numpy(x @ d.T).half().double().numpy()
    rss = np.sqrt((x ** 2) @ (w ** 2).T + wl.scale ** 2 * (h ** 2) @ (u ** 2).T)
    tol = oracle.tolerance_sum(ref, rss, oracle.F16, wl.K + wl.r)
    fin = np.isfinite(ref) & np.isfinite(g)
    err = np.abs(g - ref)
    assert (err[fin] <= tol[fin]).all(), np.argwhere(fin & (err > tol))[:5]


def test_unaligned_output_rows():
    """y that is a view starting one element into a buffer: only element alignment."""
    wl = BASE["lora_f16_4096x3072x3072_r16"].resized(M=33, N=64, K=64, r=16)
    inputs = WL.generate(wl)
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inputs.items()}
    buf = torch.zeros(33 * 64 + 1, dtype=torch.float16, device=dev)
    out = buf[1:].view(33, 64)
    say("unaligned y")
    L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, out=out)
    ref, _, _ = gpu_forward(inputs, wl)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), ref)
    assert buf[0].item() == 0


@pytest.mark.parametrize("name,dims,ksplit", [
    ("lora_bf16_16384x8192x8192_r128", dict(M=300, N=400, K=520), 2),   # 64x64 tiles, K split 2
    ("lora_f16_4096x3072x3072_r16", dict(M=16), 5),                       # decode-sized M, K split 5
])
def test_deterministic(name, dims, ksplit):
    """Bitwise-identical results on repeated calls, also where the GEMM splits
    K over several workgroups (fp32 partial sums reduced in split order by a
    second kernel) and where the h pass's guard appends elements to its work
    list with LDS atomics (each listed element is re-evaluated on its own, so
    the list's order does not reach the result)."""
    wl = BASE[name].resized(**dims)
    c_dt = L.resolve_dtypes([wl.x_dt, wl.w_dt] + ([wl.b_dt] if wl.b_dt else []) + [wl.w_dt, wl.w_dt])[0]
    r_pad = 16 if wl.r <= 16 else 128
    assert L.gemm_plan(wl.M, wl.N, wl.K, r_pad, c_dt)[0][2] == ksplit
    inputs = WL.generate(wl)
    y1, h1, f1 = gpu_forward(inputs, wl)
    for _ in range(2):
        y2, h2, f2 = gpu_forward(inputs, wl)
        assert torch.equal(y1, y2) and np.array_equal(h1, h2) and f1 == f2


@pytest.mark.parametrize("M", [64, 192])   # one fp64 dot per element (M <= 128), the split contraction
def test_h_guard_resolves_midpoints(M):
    """h values placed exactly on fp16 rounding midpoints, or 2^-20 either side,
    behind large terms that cancel exactly in pairs (so fp32 partial sums are
    inexact): h_r must still be the correctly rounded exact value, and the
    guard must have re-evaluated the elements on the midpoints."""
    K, r = 64, 16
    rng = np.random.default_rng(5)
    x = np.zeros((M, K))
    down = np.zeros((r, K))
    down[:, 0] = 1 + rng.integers(0, 1024, size=r) / 1024      # fp16 values in [1, 2)
    x[:, 0] = 1
    down[:, 1] = 2.0 ** -11                                     # + half an ulp: on the midpoint
    x[:, 1] = 1
    down[:, 2] = 2.0 ** -20                                     # a hair below, on, or above it
    x[:, 2] = rng.choice([-1.0, 0.0, 1.0], size=M)
    for k in range(3, K - 1, 2):
        v = rng.integers(1, 64, size=r) * 4.0
        u = rng.integers(1, 64, size=M) / 4.0
        down[:, k], down[:, k + 1] = v, -v
        x[:, k] = x[:, k + 1] = u
    wl = BASE["lora_f16_4096x3072x3072_r16"].resized(M=M, N=32, K=K, r=r)
    inputs = WL.generate(wl)
    inputs["x"] = torch.from_numpy(x).half()
    inputs["down"] = torch.from_numpy(down).half()
    assert np.array_equal(inputs["x"].double().numpy(), x) and np.array_equal(inputs["down"].double().numpy(), down)
    _check(wl, inputs=inputs)
    _, _, flagged = gpu_forward(inputs, wl)
    on_mid = int((x[:, 2] == 0).sum()) * r   # these rows' h sit exactly on a midpoint
    assert flagged >= on_mid > 0, (flagged, on_mid)


@pytest.mark.parametrize("M", [96, 160])   # one fp64 dot per element (M <= 128), the split contraction
@pytest.mark.parametrize("shift", [58, 62, 66])
def test_h_exact_near_fp32_underflow(shift, M):
    """bf16 x and down scaled by 2^-shift, so that the h products sit near and
    below fp32's smallest normal 2^-126 (and h itself, at the largest shift,
    in bf16's subnormal range): h_r must still be the correctly rounded exact
    value however the fp32 MFMA partial sums treat values that small."""
    wl = BASE["lora_bf16_16384x8192x8192_r128"].resized(M=M, N=64, K=640, r=16)
    inputs = WL.generate(wl)
    for k in ("x", "down"):
        inputs[k] = (inputs[k].double() * 2.0 ** -shift).to(torch.bfloat16)
    _check(wl, inputs=inputs)


# ---- the full-size workloads, in the launch configuration the benchmark uses -----

FULL = ["affine_f16_1024x768x1024", "lora_f16_4096x3072x3072_r16", "lora_bf16x_f32w_8192x4096x4096_r64",
        "lora_bf16_16384x8192x8192_r128"] + WL.SWEEP


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    wl = BASE[name]
    if (wl.x_dt, wl.w_dt) in ((1, 2), (2, 1)):
        inputs = WL.generate(wl.resized(M=8))
        with pytest.raises(L.MixedHalfError):
            gpu_forward(inputs, wl.resized(M=8))
        return
    rows = sample_rows(wl.M, 24 if wl.M * wl.N * wl.K > 1e11 else 48, seed=wl.seed)
    _check(wl, rows=rows)


# every output row of the four configurations (the oracle on the host's cores:
# about 40 s for the 16384 x 8192 x 8192 one), element by element
@pytest.mark.parametrize("name", FULL[:4])
def test_full_size_all_rows(name):
    _check(BASE[name])


@pytest.mark.parametrize("dims", [
    dict(),                                    # W split beforehand: 256 tiles of 64 x 64
    dict(M=1000, N=1100, K=520),               # ragged tiles
    dict(M=16),                                # W split inside the one contraction: nothing prepared
    dict(M=1000, N=1100, K=520, w_dt=WL.F32),  # fp32 W: its fp16 copy prepared too (fp32 y: no guard)
])
def test_prepared_weight_gives_identical_output(dims):
    """lyc_linear_prepare once, then lyc_linear_fwd_prepared (two calls, a
    second x) against lyc_linear_fwd: y bit for bit and the same guard counts."""
    wl = BASE["affine_f16_1024x768x1024"].resized(**dims)
    inputs = WL.generate(wl)
    x2 = WL.generate(wl.resized(seed=wl.seed + 7))["x"]
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inputs.items()}
    x, w, b = d["x"], d["w"], d.get("b")
    say("prepared weight", wl.name, dims)
    args = (wl.M, wl.N, wl.K, L.dtype_code(x), L.dtype_code(w), L.dtype_code(b) if b is not None else 0)
    fo, ns = L.linear_workspace_layout(*args)
    counts = lambda ws: int(ws[fo: fo + 4 * ns].cpu().view(torch.int32).sum().item()) if ns else 0
    for xx in (x, x2.to(dev)):
        ws0 = torch.empty(max(L.linear_workspace_size(*args), 1), dtype=torch.uint8, device=dev)
        y0 = L.linear(xx, w, b, workspace=ws0)
        ws1 = L.linear_prepare(w, wl.M, xx.dtype, b.dtype if b is not None else None)
        y1 = L.linear(xx, w, b, workspace=ws1, prepared=True)
        y2 = L.linear(xx, w, b, workspace=ws1, prepared=True)
        y3 = L.linear(xx, w, b, workspace=ws0, prepared=True)   # a plain call's workspace is prepared too
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(y0, y2) and torch.equal(y0, y3)
        assert counts(ws0) == counts(ws1)


@pytest.mark.parametrize("name,dims", [
    ("lora_bf16x_f32w_8192x4096x4096_r64", dict(M=257, N=200, K=264)),   # fp32 W, factors and y under bf16
    ("sweep_xf32_wf32_2048x1280x5120_r32", dict(M=130, N=96, K=136)),    # fp32 x still cast per call
    ("lora_bf16_16384x8192x8192_r128", dict(M=270, N=300, K=520)),       # 16-bit W: W_c is W itself
    ("lora_bf16x_f32w_8192x4096x4096_r64", dict()),                      # full size
])
def test_kept_compute_copy_gives_identical_output(name, dims):
    """lyc_lora_linear_fwd_wc (W rounded to the compute dtype once, by the
    caller) against lyc_lora_linear_fwd: y and h_r bit for bit."""
    wl = BASE[name].resized(**dims) if dims else BASE[name]
    inputs = WL.generate(wl)
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inputs.items()}
    codes = [WL.dtype_code(inputs[k]) for k in ("x", "w", "down", "up")] + \
            ([WL.dtype_code(inputs["b"])] if "b" in inputs else [])
    c_dt, _ = L.resolve_dtypes(codes)
    w_c = d["w"].to(L.torch_dtype(c_dt)).contiguous()
    say("kept compute copy", wl.name, dims)
    y0, ws0 = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), return_workspace=True)
    y1, ws1 = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"), return_workspace=True,
                            w_c=w_c)
    h0 = L.lora_saved_h(ws0, d["x"], d["w"], d["down"], d["up"], d.get("b"))
    h1 = L.lora_saved_h(ws1, d["x"], d["w"], d["down"], d["up"], d.get("b"))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.equal(h0, h1)
