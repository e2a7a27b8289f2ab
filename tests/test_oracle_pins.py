"""Pins for the CPU oracle: checks against what the pages and mathematics fix,
never against the oracle itself or the GPU path.

Covers: rounding (exhaustive round trips, every midpoint, library conversions,
overflow and subnormal edges, direct-from-fp64 rounding), the dtype-policy
table, the hand-built boundary fixtures, exact-rational brute force on tiny
shapes, closed forms and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact
from tests.exact import BF16, F16, F32

# ---- rounding ------------------------------------------------------------------


def _all_finite(dt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        if dt == F16:
            vals = bits.view(np.float16).astype(np.float64)
        else:
            vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    keep = np.isfinite(vals)
    return bits[keep], vals[keep]


@pytest.mark.parametrize("dt", [F16, BF16])
def test_roundtrip_every_16bit_pattern(dt):
    bits, vals = _all_finite(dt)
    # widening agrees with the library decode of every pattern
    np.testing.assert_array_equal(oracle.widen(bits, dt), vals)
    # rounding a representable value is the identity, and storing it restores the pattern
    np.testing.assert_array_equal(oracle.round_array(vals, dt), vals)
    np.testing.assert_array_equal(oracle.encode(vals, dt), bits)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_every_midpoint_ties_to_even(dt):
    bits, vals = _all_finite(dt)
    pos = np.unique(vals[vals >= 0])
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2                      # exact in fp64
    got = oracle.round_array(mid, dt)
    even_lo = (oracle.encode(lo, dt) & 1) == 0
    np.testing.assert_array_equal(got, np.where(even_lo, lo, hi))
    np.testing.assert_array_equal(oracle.round_array(-mid, dt), -np.where(even_lo, lo, hi))
    # one fp64 step either side of the midpoint goes to the nearer neighbour
    np.testing.assert_array_equal(oracle.round_array(np.nextafter(mid, -np.inf), dt), lo)
    np.testing.assert_array_equal(oracle.round_array(np.nextafter(mid, np.inf), dt), hi)


def test_fp16_matches_numpy_direct_conversion():
    # numpy converts binary64 -> binary16 directly with round-to-nearest-even
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.uniform(-9, 5, 200000),
                        np.array([65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -25, 2.0 ** -25 * 1.0000001,
                                  3 * 2.0 ** -26, 2.0 ** -24, 6e-8, 0.0, -0.0])])
    with np.errstate(over="ignore"):
        lib = v.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_array(v, F16), lib)


def test_fp32_matches_c_conversion():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(200000) * 10.0 ** rng.uniform(-46, 39, 200000)
    v = np.concatenate([v, [3.4028235677973366e38, 3.4028235677973362e38, 2.0 ** -149, 2.0 ** -150,
                            2.0 ** -150 * 1.5, 1.401298464324817e-45]])
    with np.errstate(over="ignore"):
        lib = v.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_array(v, F32), lib)


def test_bf16_matches_torch_on_fp32_inputs():
    # torch rounds fp32 -> bf16 to nearest even; on fp32 inputs no double rounding is involved
    rng = np.random.default_rng(2)
    v32 = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-40, 38, 200000)).astype(np.float32)
    lib = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_array(v32.astype(np.float64), BF16), lib)


def test_overflow_thresholds():
    # overflow to inf at or beyond max + half an ulp (ties go to the even "next" value)
    assert oracle.round_to(65504.0 + 16.0, F16) == np.inf
    assert oracle.round_to(np.nextafter(65504.0 + 16.0, 0), F16) == 65504.0
    bmax = float(torch.finfo(torch.bfloat16).max)
    half_ulp = 2.0 ** (127 - 8)
    assert oracle.round_to(bmax + half_ulp, BF16) == np.inf
    assert oracle.round_to(np.nextafter(bmax + half_ulp, 0), BF16) == bmax
    assert oracle.round_to(-(bmax + half_ulp), BF16) == -np.inf
    assert np.isnan(oracle.round_to(np.nan, F16))


def test_rounds_directly_from_fp64_not_via_fp32():
    # 1 + 2^-8 + 2^-30: bf16 neighbours 1 and 1 + 2^-7, midpoint 1 + 2^-8; the value is just above it.
    # Going through fp32 first loses the 2^-30 and lands on the midpoint, which ties down to 1.
    v = 1 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.round_to(v, BF16) == 1 + 2.0 ** -7
    assert float(torch.tensor(v, dtype=torch.float64).to(torch.float32).to(torch.bfloat16)) == 1.0


def test_subnormals_kept():
    assert oracle.round_to(2.0 ** -20, F16) == 2.0 ** -20           # fp16 subnormal
    assert oracle.round_to(2.0 ** -25, F16) == 0.0                  # half of the smallest: ties to even (0)
    assert oracle.round_to(3 * 2.0 ** -26, F16) == 2.0 ** -24
    assert oracle.round_to(2.0 ** -133, BF16) == 2.0 ** -133        # smallest bf16 subnormal


# ---- dtype policy -------------------------------------------------------------


def test_policy_table_exact():
    for x_dt, w_dt, c_dt, o_dt in exact.load_policy_table():
        # the module weights W, b, down, up share w_dt
        st, c, o = oracle.resolve([x_dt, w_dt, w_dt, w_dt, w_dt])
        if c_dt is None:
            assert st == oracle.MIXED_HALF
        else:
            assert (st, c, o) == (oracle.OK, c_dt, o_dt)


_TORCH = {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}
_BACK = {v: k for k, v in _TORCH.items()}


def test_policy_every_operand_tuple():
    """All 3^5 operand tuples: output is torch's type promotion over the
    operands; rejection exactly when both 16-bit types are present; compute is
    the 16-bit type present, else fp32."""
    import itertools
    for tup in itertools.product([F16, BF16, F32], repeat=5):
        st, c, o = oracle.resolve(list(tup))
        if F16 in tup and BF16 in tup:
            assert st == oracle.MIXED_HALF, tup
            continue
        prom = _TORCH[tup[0]]
        for t in tup[1:]:
            prom = torch.promote_types(prom, _TORCH[t])
        assert st == oracle.OK and o == _BACK[prom], tup
        sixteen = [t for t in tup if t != F32]
        assert c == (sixteen[0] if sixteen else F32), tup


def test_policy_invalid():
    assert oracle.resolve([])[0] == oracle.INVALID
    assert oracle.resolve([1, 7])[0] == oracle.INVALID


# ---- fixtures -----------------------------------------------------------------

FIXTURES = exact.load_fixtures()


def _run_fixture(fx):
    a = exact.fixture_arrays(fx)
    dt = a["dt"]
    lora = fx["kind"] == "lora"
    res = oracle.forward(a["x"], dt, a["w"], dt, a["b"], dt if a["b"] is not None else None,
                         a.get("down"), dt if lora else None, a.get("up"), dt if lora else None,
                         scale=a.get("scale", 1.0), lora=lora, nthreads=1)
    return a, res


@pytest.mark.parametrize("fx", FIXTURES, ids=[f["name"] for f in FIXTURES])
def test_fixture_oracle_value(fx):
    a, res = _run_fixture(fx)
    y = oracle.as_float64(res["y"], res["output"])[0, 0]
    assert Fraction(float(y)) == fx["expect"], (fx["name"], y, float(fx["expect"]))


@pytest.mark.parametrize("fx", FIXTURES, ids=[f["name"] for f in FIXTURES])
def test_fixture_has_teeth(fx):
    """Every named wrong implementation falls outside the tolerance."""
    dt = {"f16": F16, "bf16": BF16}[fx["dtype"]]
    ref = np.array([float(fx["expect"])])
    tol = oracle.tolerance(ref, dt, 8, 1)[0]
    for wrong, what in fx["wrong"]:
        assert abs(float(wrong) - float(fx["expect"])) > tol, (fx["name"], what)


@pytest.mark.parametrize("fx", FIXTURES, ids=[f["name"] for f in FIXTURES])
def test_fixture_exact_rational(fx):
    """The hand-derived expectation is what exact rational evaluation gives."""
    a = exact.fixture_arrays(fx)
    dt = a["dt"]
    lora = fx["kind"] == "lora"
    y, _ = exact.exact_forward(a["x"], dt, a["w"], dt, dt, dt, b=a["b"], b_dt=dt, down=a.get("down"), d_dt=dt,
                               up=a.get("up"), u_dt=dt, scale=Fraction(a.get("scale", 1.0)), lora=lora)
    assert y[0][0] == fx["expect"]


# ---- exact-rational brute force -------------------------------------------------

def _draw(rng, shape, dt, std=1.0):
    v = (rng.standard_normal(shape) * std).astype(np.float32)
    return {F16: lambda: v.astype(np.float16).view(np.uint16),
            BF16: lambda: torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16),
            F32: lambda: v}[dt]()


CASES = [  # (x_dt, w_dt, M, N, K, r)
    (F16, F16, 4, 4, 8, 1), (F16, F16, 4, 4, 8, 2), (F16, F16, 4, 4, 8, 4),
    (BF16, BF16, 4, 4, 8, 2), (BF16, BF16, 3, 5, 7, 3),
    (F16, F32, 3, 5, 7, 1), (F32, BF16, 3, 5, 7, 2), (BF16, F32, 4, 4, 8, 4), (F32, F32, 3, 4, 8, 2),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_lora_exact(case, seed):
    x_dt, w_dt, M, N, K, r = case
    rng = np.random.default_rng(100 + seed)
    x = _draw(rng, (M, K), x_dt)
    w = _draw(rng, (N, K), w_dt, 0.5)
    b = _draw(rng, (N,), w_dt, 0.3)
    down = _draw(rng, (r, K), w_dt, 0.5)
    up = _draw(rng, (N, r), w_dt, 0.5)
    scale = [1.0, 0.5, 3.0][seed]
    res = oracle.forward(x, x_dt, w, w_dt, b, w_dt, down, w_dt, up, w_dt, scale=scale, nthreads=2)
    y, hr = exact.exact_forward(x, x_dt, w, w_dt, res["compute"], res["output"], b=b, b_dt=w_dt, down=down,
                                d_dt=w_dt, up=up, u_dt=w_dt, scale=Fraction(scale))
    got = oracle.as_float64(res["y"], res["output"])
    for m in range(M):
        for j in range(r):
            assert Fraction(float(res["h"][m, j])) == hr[m][j]
        for n in range(N):
            assert Fraction(float(got[m, n])) == y[m][n], (m, n)


@pytest.mark.parametrize("dt", [F16, BF16, F32])
def test_bruteforce_linear_exact(dt):
    rng = np.random.default_rng(7)
    M, N, K = 4, 4, 8
    x, w, b = _draw(rng, (M, K), dt), _draw(rng, (N, K), dt, 0.4), _draw(rng, (N,), dt, 0.2)
    res = oracle.forward(x, dt, w, dt, b, dt, lora=False, nthreads=1)
    y, _ = exact.exact_forward(x, dt, w, dt, dt, dt, b=b, b_dt=dt, lora=False)
    got = oracle.as_float64(res["y"], res["output"])
    for m in range(M):
        for n in range(N):
            assert Fraction(float(got[m, n])) == y[m][n]


# ---- closed forms and invariants -------------------------------------------------

def _medium(seed, dt=F16, M=24, N=40, K=96, r=8):
    rng = np.random.default_rng(seed)
    return (_draw(rng, (M, K), dt), _draw(rng, (N, K), dt, K ** -0.5), _draw(rng, (N,), dt, 0.3),
            _draw(rng, (r, K), dt, K ** -0.5), _draw(rng, (N, r), dt, r ** -0.5))


def _np_vals(a, dt):
    return oracle.as_float64(a, dt)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_closed_form_zero_bypass(dt):
    """down = 0, up = 0 or scale = 0: y = round(x.W^T + b), a single rounding,
    computed here with numpy's fp64 matmul and numpy/torch rounding."""
    x, w, b, down, up = _medium(11, dt)
    X, Wv, Bv = _np_vals(x, dt), _np_vals(w, dt), _np_vals(b, dt)
    expect = X @ Wv.T + Bv
    if dt == F16:
        expect_r = expect.astype(np.float16).astype(np.float64)
    else:
        expect_r = oracle.round_array(expect, BF16)  # checked against torch below
        np.testing.assert_array_equal(expect_r[np.abs(expect_r) > 0],
                                      torch.from_numpy(expect).to(torch.float32).to(torch.bfloat16)
                                      .to(torch.float64).numpy()[np.abs(expect_r) > 0])
    zeros_d = np.zeros_like(down)
    zeros_u = np.zeros_like(up)
    for d_, u_, s_ in ((zeros_d, up, 1.0), (down, zeros_u, 1.0), (down, up, 0.0)):
        res = oracle.forward(x, dt, w, dt, b, dt, d_, dt, u_, dt, scale=s_)
        np.testing.assert_array_equal(oracle.as_float64(res["y"], dt), expect_r)


def test_closed_form_zero_weight_f16():
    """W = 0: y = round(scale * h_r.up^T + b) with h_r = round(x.down^T)."""
    x, w, b, down, up = _medium(12, F16)
    X, D, U, Bv = (_np_vals(a, F16) for a in (x, down, up, b))
    h_r = (X @ D.T).astype(np.float16).astype(np.float64)
    expect = (2.0 * (h_r @ U.T) + Bv).astype(np.float16).astype(np.float64)
    res = oracle.forward(x, F16, np.zeros_like(w), F16, b, F16, down, F16, up, F16, scale=2.0)
    np.testing.assert_array_equal(res["h"], h_r)
    np.testing.assert_array_equal(oracle.as_float64(res["y"], F16), expect)


def test_closed_form_unit_rows():
    """x = e_k: h = down[:, k] exactly, so h_r = down[:, k]."""
    K, r = 16, 4
    x = np.zeros((K, K), dtype=np.float16)
    np.fill_diagonal(x, 1.0)
    x = x.view(np.uint16)
    _, w, b, down, up = _medium(13, F16, M=K, N=8, K=K, r=r)
    res = oracle.forward(x, F16, w, F16, b, F16, down, F16, up, F16, scale=1.0)
    np.testing.assert_array_equal(res["h"], _np_vals(down, F16).T)


@pytest.mark.parametrize("k", [-3, 2])
def test_invariant_power_of_two_scaling(k):
    """With b = 0, scaling x by 2^k scales y (and h) by 2^k exactly in the normal range."""
    x, w, b, down, up = _medium(14, F16)
    x2 = (_np_vals(x, F16) * 2.0 ** k).astype(np.float16).view(np.uint16)
    r1 = oracle.forward(x, F16, w, F16, None, None, down, F16, up, F16, scale=1.0)
    r2 = oracle.forward(x2, F16, w, F16, None, None, down, F16, up, F16, scale=1.0)
    y1, y2 = oracle.as_float64(r1["y"], F16), oracle.as_float64(r2["y"], F16)
    normal = (np.abs(y1) >= 2.0 ** -14 * 2 ** max(0, -k)) & (np.abs(y1) * 2.0 ** k < 32768)
    assert normal.mean() > 0.9
    np.testing.assert_array_equal(y2[normal], y1[normal] * 2.0 ** k)


def test_invariant_consistent_k_permutation():
    x, w, b, down, up = _medium(15, F16)
    perm = np.random.default_rng(3).permutation(x.shape[1])
    r1 = oracle.forward(x, F16, w, F16, b, F16, down, F16, up, F16, scale=1.0)
    r2 = oracle.forward(x[:, perm], F16, w[:, perm], F16, b, F16, down[:, perm], F16, up, F16, scale=1.0)
    np.testing.assert_array_equal(r1["y"], r2["y"])
    np.testing.assert_array_equal(r1["h"], r2["h"])


def test_rows_subset_matches_full():
    x, w, b, down, up = _medium(16, BF16)
    full = oracle.forward(x, BF16, w, BF16, b, BF16, down, BF16, up, BF16, scale=0.5)
    rows = np.array([3, 0, 23, 11])
    part = oracle.forward(x, BF16, w, BF16, b, BF16, down, BF16, up, BF16, scale=0.5, rows=rows)
    np.testing.assert_array_equal(part["y"], full["y"][rows])
    np.testing.assert_array_equal(part["ref"], full["ref"][rows])


def test_mixed_half_rejected_by_forward():
    x, w, b, down, up = _medium(17, F16)
    with pytest.raises(oracle.OracleError):
        oracle.forward(x, F16, w, BF16, None, None, down, BF16, up, BF16)


# ---- the LoRA merge W' = round_out(W + scale * up_c . down_c) ------------------------

def _exact_merge(w, w_dt, down, up, m_dt, c_dt, o_dt, scale):
    """The merge in exact rational arithmetic: W keeps its stored value, up and
    down are rounded to the compute dtype, one rounding at the end."""
    N, K = w.shape
    r = down.shape[0]
    W = exact.to_fraction_array(w, w_dt)
    D = [exact.exact_round(v, c_dt) for v in exact.to_fraction_array(down, m_dt)]
    U = [exact.exact_round(v, c_dt) for v in exact.to_fraction_array(up, m_dt)]
    return [[exact.exact_round(W[n * K + k] + scale * sum(U[n * r + j] * D[j * K + k] for j in range(r)), o_dt)
             for k in range(K)] for n in range(N)]


MERGE_CASES = [  # (W dtype, module dtype, N, K, r)
    (F16, F16, 4, 8, 1), (F16, F16, 3, 7, 4), (BF16, BF16, 4, 6, 2), (F32, F32, 3, 5, 3),
    (F32, F16, 4, 5, 2), (F32, BF16, 3, 6, 4), (F16, F32, 3, 5, 2),
]


@pytest.mark.parametrize("case", MERGE_CASES)
@pytest.mark.parametrize("seed", [0, 1])
def test_bruteforce_merge_exact(case, seed):
    w_dt, m_dt, N, K, r = case
    rng = np.random.default_rng(300 + seed)
    w = _draw(rng, (N, K), w_dt, 0.5)
    down = _draw(rng, (r, K), m_dt, 0.5)
    up = _draw(rng, (N, r), m_dt, 0.5)
    scale = [1.0, 0.75][seed]
    res = oracle.merge(w, w_dt, down, m_dt, up, m_dt, scale=scale, nthreads=2)
    want = _exact_merge(w, w_dt, down, up, m_dt, res["compute"], res["output"], Fraction(scale))
    got = oracle.as_float64(res["y"], res["output"])
    for n in range(N):
        for k in range(K):
            assert Fraction(float(got[n, k])) == want[n][k], (n, k)


def test_merge_policy():
    w = _draw(np.random.default_rng(1), (2, 3), F16)
    d = _draw(np.random.default_rng(2), (1, 3), BF16)
    u = _draw(np.random.default_rng(3), (2, 1), BF16)
    with pytest.raises(oracle.OracleError):
        oracle.merge(w, F16, d, BF16, u, BF16)
    # an fp32 master weight with fp16 modules: fp16 compute, fp32 result
    w32 = _draw(np.random.default_rng(4), (2, 3), F32)
    d16, u16 = _draw(np.random.default_rng(5), (1, 3), F16), _draw(np.random.default_rng(6), (2, 1), F16)
    res = oracle.merge(w32, F32, d16, F16, u16, F16)
    assert (res["compute"], res["output"]) == (F16, F32)


@pytest.mark.parametrize("w_dt,m_dt", [(F16, F16), (BF16, BF16), (F32, F16), (F32, F32)])
def test_merge_closed_form_zero_bypass(w_dt, m_dt):
    rng = np.random.default_rng(11)
    w = _draw(rng, (6, 10), w_dt)
    down = _draw(rng, (3, 10), m_dt)
    up = _draw(rng, (6, 3), m_dt)
    zero_up = np.zeros_like(up)
    for args in ((down, up, 0.0), (down, zero_up, 1.5)):
        res = oracle.merge(w, w_dt, args[0], m_dt, args[1], m_dt, scale=args[2])
        # the weight is returned unchanged (it is exactly representable in the result dtype)
        np.testing.assert_array_equal(oracle.as_float64(res["y"], res["output"]), oracle.as_float64(w, w_dt))


def test_merge_fixture_single_rounding():
    # W = 1, up . down = 2^-11 + 2^-22 exactly: the sum lies just above the fp16
    # midpoint 1 + 2^-11 and rounds up; rounding the product to fp16 first
    # (2^-11 + 2^-22 is itself a tie and goes to 2^-11) would land on the tie and give 1
    w = oracle.encode([1.0], F16).reshape(1, 1)
    down = oracle.encode([2.0 ** -11, 2.0 ** -22], F16).reshape(2, 1)
    up = oracle.encode([1.0, 1.0], F16).reshape(1, 2)
    res = oracle.merge(w, F16, down, F16, up, F16)
    assert float(oracle.as_float64(res["y"], F16)[0, 0]) == 1.0 + 2.0 ** -10
    early = oracle.round_to(1.0 + oracle.round_to(2.0 ** -11 + 2.0 ** -22, F16), F16)
    assert early == 1.0


def test_merge_invariants():
    rng = np.random.default_rng(12)
    w, down, up = _draw(rng, (8, 12), BF16), _draw(rng, (5, 12), BF16, 0.3), _draw(rng, (8, 5), BF16, 0.3)
    full = oracle.merge(w, BF16, down, BF16, up, BF16, scale=2.0)
    perm = np.array([3, 0, 4, 1, 2])
    # the rank index permuted consistently in up and down (random non-tie inputs)
    pm = oracle.merge(w, BF16, down[perm], BF16, up[:, perm], BF16, scale=2.0)
    np.testing.assert_array_equal(pm["y"], full["y"])
    rows = np.array([7, 2, 2, 0])
    part = oracle.merge(w, BF16, down, BF16, up, BF16, scale=2.0, rows=rows)
    np.testing.assert_array_equal(part["y"], full["y"][rows])


# ---- scoring --------------------------------------------------------------------

def test_tolerance_constants_from_pages():
    # abs(actual-reference) <= 2e-4 + 2e-3*abs(reference) (Luminal FP16 page)
    assert oracle.tolerance(np.array([0.0, 1.0, -10.0]), F16, 64, 0).tolist() == [2e-4, 2e-4 + 2e-3, 2e-4 + 2e-2]


def test_ulp_report():
    ref = np.array([1.0, -1.0, 1.0, -1.0])
    act = ref + np.array([2.0 ** -10, 0, 0, 2.0 ** -11])     # fp16 ulp at RMS 1 is 2^-10
    mx, rms = oracle.ulp_report(act, ref, F16)
    assert mx == 1.0 and rms == pytest.approx(np.sqrt((1 + 0.25) / 4))
    assert oracle.ulp_of(1.0, BF16) == 2.0 ** -7
    assert oracle.ulp_of(1.0, F32) == 2.0 ** -23


# ---- the backward ------------------------------------------------------------------
#
# Pinned against the forward map itself: for y = x W^T + scale (x down^T) up^T
# the loss L = sum(dy * y) is linear in each of x, down and up when the other
# two are held, so every partial derivative is exactly L(theta + e_i) - L(theta).
# With small-integer inputs nothing rounds anywhere (h, gh and every gradient
# are exact in the storage dtype), so the oracle's gradients must equal these
# exact differences bit for bit.  That pins which operand meets which, every
# transpose and where scale enters, independently of the backward formula.


def _int_draw(rng, shape, lim, dt):
    v = rng.integers(-lim, lim + 1, size=shape).astype(np.float64)
    return oracle.encode(v.ravel(), dt).reshape(shape), v


def _loss(x, w, down, up, dy, scale):
    """sum(dy * y) of the unrounded forward, in exact rationals."""
    M, K = x.shape
    N, r = up.shape
    L = Fraction(0)
    for m in range(M):
        h = [sum(Fraction(x[m, k]) * Fraction(down[j, k]) for k in range(K)) for j in range(r)]
        for n in range(N):
            y = sum(Fraction(x[m, k]) * Fraction(w[n, k]) for k in range(K))
            y += scale * sum(h[j] * Fraction(up[n, j]) for j in range(r))
            L += Fraction(dy[m, n]) * y
    return L


def _exact_grad(theta, bump):
    """Partial derivatives of a function linear in theta: f(theta + e_i) - f(theta)."""
    base = bump(theta)
    g = np.zeros(theta.shape)
    for idx in np.ndindex(*theta.shape):
        t = theta.copy()
        t[idx] += 1
        g[idx] = float(bump(t) - base)
    return g


BWD_EXACT = [  # (dtype, lim, scale, M, N, K, r)
    (F16, 3, Fraction(1, 2), 3, 4, 5, 2), (F16, 2, Fraction(2), 2, 3, 4, 3),
    (BF16, 1, Fraction(1, 2), 3, 4, 5, 2), (F32, 3, Fraction(3, 4), 3, 3, 4, 2),
]


@pytest.mark.parametrize("case", BWD_EXACT)
def test_backward_is_the_exact_gradient_of_the_forward(case):
    dt, lim, scale, M, N, K, r = case
    rng = np.random.default_rng(M * 7 + r)
    xs, x = _int_draw(rng, (M, K), lim, dt)
    ws, w = _int_draw(rng, (N, K), lim, dt)
    ds, d = _int_draw(rng, (r, K), lim, dt)
    us, u = _int_draw(rng, (N, r), lim, dt)
    gs, g = _int_draw(rng, (M, N), lim, dt)
    res = oracle.backward(xs, dt, ws, dt, ds, dt, us, dt, gs, dt, scale=float(scale))
    want_dx = _exact_grad(x, lambda t: _loss(t, w, d, u, g, scale))
    want_dd = _exact_grad(d, lambda t: _loss(x, w, t, u, g, scale))
    want_du = _exact_grad(u, lambda t: _loss(x, w, d, t, g, scale))
    np.testing.assert_array_equal(oracle.as_float64(res["dx"], dt), want_dx)
    np.testing.assert_array_equal(oracle.as_float64(res["d_down"], dt), want_dd)
    np.testing.assert_array_equal(oracle.as_float64(res["d_up"], dt), want_du)
    assert np.any(want_dd != 0) and np.any(want_du != 0)


def test_backward_gh_rounded_once_fixture():
    """fp16, M = K = r = 1, N = 2.  gh = scale * dy.up = 1 + 2^-11 + 2^-20 lies
    just above the midpoint 1 + 2^-11 and rounds to gh_r = 1 + 2^-10; then
    dx = dy.W + gh_r.down = (-1 - 2^-10) + (1 + 2^-10) = 0 exactly.  Without
    the rounding of gh, dx would be -2^-11 + 2^-20 (-4.87e-4, beyond the fp16
    bound 2e-4 of the Luminal page); with gh truncated, -2^-10."""
    enc = lambda v, s: oracle.encode(np.array(v, dtype=np.float64).ravel(), F16).reshape(s)
    x, w = enc([1.0], (1, 1)), enc([-1.0, -(2.0 ** -10)], (2, 1))
    down, up = enc([1.0], (1, 1)), enc([1.0, 2.0 ** -11 + 2.0 ** -20], (2, 1))
    dy = enc([1.0, 1.0], (1, 2))
    res = oracle.backward(x, F16, w, F16, down, F16, up, F16, dy, F16, scale=1.0)
    assert res["gh"][0, 0] == 1.0 + 2.0 ** -10
    assert oracle.as_float64(res["dx"], F16)[0, 0] == 0.0
    assert oracle.as_float64(res["d_down"], F16)[0, 0] == 1.0 + 2.0 ** -10     # gh_r . x
    assert oracle.as_float64(res["d_up"], F16)[:, 0].tolist() == [1.0, 1.0]     # dy^T . h_r, h_r = 1
    unrounded = -1.0 - 2.0 ** -10 + 1.0 + 2.0 ** -11 + 2.0 ** -20
    assert abs(unrounded) > oracle.tolerance(np.array([0.0]), F16, 2, 1)[0]


@pytest.mark.parametrize("dt", [F16, BF16, F32])
def test_backward_closed_forms(dt):
    rng = np.random.default_rng(21)
    M, N, K, r = 5, 6, 8, 3
    x, w, d, u, g = (_draw(rng, s, dt, 0.5) for s in ((M, K), (N, K), (r, K), (N, r), (M, N)))
    # dx with no bypass is the plain product dy . W: the (pinned) forward of dy with W^T
    wt = np.ascontiguousarray(w.reshape(N, K).T)
    plain = oracle.forward(g, dt, wt, dt, None, None, None, None, None, None, lora=False)["y"]
    for kw in (dict(scale=0.0, up=np.zeros_like(u)), dict(scale=1.5, up=np.zeros_like(u))):
        res = oracle.backward(x, dt, w, dt, d, dt, kw["up"], dt, g, dt, scale=kw["scale"])
        np.testing.assert_array_equal(res["dx"], plain)
        assert not np.any(oracle.as_float64(res["d_down"], dt))
    res = oracle.backward(x, dt, w, dt, d, dt, u, dt, g, dt, scale=0.0)
    np.testing.assert_array_equal(res["dx"], plain)
    assert not np.any(oracle.as_float64(res["d_up"], dt)) and not np.any(oracle.as_float64(res["d_down"], dt))
    res = oracle.backward(x, dt, w, dt, np.zeros_like(d), dt, u, dt, g, dt, scale=1.5)   # h = 0
    assert not np.any(oracle.as_float64(res["d_up"], dt))


def test_backward_recomputes_the_forward_h():
    """With dy = e_(m,n) and scale 1, dUp[n, :] = h_r[m, :]: the forward's rounded h."""
    rng = np.random.default_rng(22)
    M, N, K, r = 4, 3, 16, 4
    x, w, d, u = (_draw(rng, s, BF16) for s in ((M, K), (N, K), (r, K), (N, r)))
    h = oracle.forward(x, BF16, w, BF16, None, None, d, BF16, u, BF16, scale=1.0)["h"]
    for m, n in ((0, 0), (3, 2), (2, 1)):
        g = np.zeros((M, N))
        g[m, n] = 1.0
        res = oracle.backward(x, BF16, w, BF16, d, BF16, u, BF16, oracle.encode(g.ravel(), BF16).reshape(M, N),
                              BF16, scale=1.0)
        np.testing.assert_array_equal(oracle.as_float64(res["d_up"], BF16)[n], h[m])


def test_backward_invariants_and_subsets():
    rng = np.random.default_rng(23)
    M, N, K, r = 6, 5, 16, 3
    dt = F16
    x, w, d, u, g = (_draw(rng, s, dt, 0.5) for s in ((M, K), (N, K), (r, K), (N, r), (M, N)))
    full = oracle.backward(x, dt, w, dt, d, dt, u, dt, g, dt, scale=0.75)
    # dy doubled: every gradient doubles exactly (no overflow or underflow here)
    g2 = oracle.encode(2 * oracle.as_float64(g, dt).ravel(), dt).reshape(M, N)
    dbl = oracle.backward(x, dt, w, dt, d, dt, u, dt, g2, dt, scale=0.75)
    for key in ("dx", "d_down", "d_up"):
        np.testing.assert_array_equal(oracle.as_float64(dbl[key], dt), 2 * oracle.as_float64(full[key], dt))
    # index subsets select the same values
    sub = oracle.backward(x, dt, w, dt, d, dt, u, dt, g, dt, scale=0.75, dx_rows=[5, 0, 0], js=[2, 0],
                          dd_cols=[15, 3], du_rows=[4, 1])
    np.testing.assert_array_equal(sub["dx"], full["dx"][[5, 0, 0]])
    np.testing.assert_array_equal(sub["d_down"], full["d_down"][np.ix_([2, 0], [15, 3])])
    np.testing.assert_array_equal(sub["d_up"], full["d_up"][np.ix_([4, 1], [2, 0])])


def test_backward_policy():
    rng = np.random.default_rng(24)
    M, N, K, r = 2, 3, 4, 2
    x, w = _draw(rng, (M, K), F32), _draw(rng, (N, K), F32)
    d, u = _draw(rng, (r, K), BF16), _draw(rng, (N, r), BF16)
    g = _draw(rng, (M, N), F32)
    res = oracle.backward(x, F32, w, F32, d, BF16, u, BF16, g, F32)
    assert res["compute"] == BF16
    assert res["dx"].dtype == np.float32 and res["d_down"].dtype == np.uint16 and res["d_up"].dtype == np.uint16
    assert oracle.backward(x, F32, w, F32, d, F32, u, F32, g, F32, b_dt=F16)["compute"] == F16   # the bias counts
    with pytest.raises(oracle.OracleError):
        oracle.backward(x, F32, w, F32, d, BF16, u, BF16, _draw(rng, (M, N), F16), F16)


def test_backward_mixed_dtype_fixture():
    """x, W, dy and down in fp32, up in fp16: the compute dtype is fp16.
    x = 1 + 2^-12 rounds to x_c = 1; dy = [1, 2^-12] is exact in fp16; up =
    [1, 0] gives gh_r = 1 and h_r = x_c . down_c = 1.  Then
      dx    = dy_c.W_c + gh_r.down_c = (1 + 2^-12) + 1 = 2 + 2^-12, kept in
              fp32 (x's dtype), not rounded through fp16 (which gives 2);
      dDown = gh_r . x_c = 1 (with the uncast x it would be 1 + 2^-12, and
              down's dtype fp32 would keep that);
      dUp   = dy_c^T . h_r = [1, 2^-12] in fp16."""
    f32 = lambda v, s: np.array(v, dtype=np.float32).reshape(s)
    x, w, down, dy = f32([1 + 2.0 ** -12], (1, 1)), f32([1.0, 1.0], (2, 1)), f32([1.0], (1, 1)), f32([1.0, 2.0 ** -12], (1, 2))
    up = oracle.encode(np.array([1.0, 0.0]), F16).reshape(2, 1)
    res = oracle.backward(x, F32, w, F32, down, F32, up, F16, dy, F32, scale=1.0)
    assert res["compute"] == F16
    assert res["gh"][0, 0] == 1.0
    assert float(res["dx"][0, 0]) == 2.0 + 2.0 ** -12
    assert float(res["d_down"][0, 0]) == 1.0
    assert oracle.as_float64(res["d_up"], F16)[:, 0].tolist() == [1.0, 2.0 ** -12]


def test_tolerance_sum_forms():
    # 16-bit: the forward's bound plus the fp32 accumulation term; fp32: terms' scale in place of 1
    ref, rss = np.array([0.0, 2.0]), np.array([0.0, 8.0])
    acc = 8.0 * 2.0 ** -24 * 10.0 * rss                         # sqrt(L) = 10
    np.testing.assert_allclose(oracle.tolerance_sum(ref, rss, F16, 100), 2e-4 + 2e-3 * ref + acc)
    np.testing.assert_allclose(oracle.tolerance_sum(ref, rss, F32, 100), 8.0 * 2.0 ** -24 * 10.0 * ref + acc)
    # the forward's fp32 bound is the special case rss = 1
    np.testing.assert_allclose(oracle.tolerance_sum(ref, np.ones(2), F32, 100), oracle.tolerance(ref, F32, 100, 0))


# ---- DoRA ----------------------------------------------------------------------------

def test_dora_norms_exact_and_correctly_rounded():
    """Integer rows whose merged norms are exact (3, 7, 9) or irrational (sqrt 18):
    the fp32 norm is the exact square root rounded once to fp32."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    enc = lambda v, dt, s: oracle.encode(np.array(v, dtype=np.float64).ravel(), dt).reshape(s)
    # W + up.down: up = [0, 0, 1, 1]^T, down = [[1, 0, 0, 0]]
    W = [[1, 2, 2, 0], [2, 3, 6, 0], [0, 4, 8, 0], [2, 3, 0, 0]]
    w, down, up = enc(W, F16, (4, 4)), enc([1, 0, 0, 0], F16, (1, 4)), enc([0, 0, 1, 1], F16, (4, 1))
    norms, exact, c = oracle.dora_norms(w, F16, down, F16, up, F16, scale=1.0)
    merged = np.array(W, dtype=np.float64) + np.outer([0, 0, 1, 1], [1, 0, 0, 0])
    for n in range(4):
        q = sum(Decimal(int(v)) ** 2 for v in merged[n])
        want = oracle.round_to(float(q.sqrt()), F32)
        assert float(norms[n]) == want, (n, norms[n], want)
    assert norms[:3].tolist() == [3.0, 7.0, 9.0] and abs(float(norms[3]) - 18 ** 0.5) < 3e-7   # [3, 3, 0, 0]


def _dora_case(dt, rng, M=5, K=8, with_bias=True):
    enc = lambda v: oracle.encode(np.asarray(v, dtype=np.float64).ravel(), dt).reshape(np.shape(v))
    rows = np.zeros((4, K))
    rows[0, :3] = [1, 2, 2]
    rows[1, :3] = [2, 3, 6]
    rows[2, :3] = [1, 4, 8]
    rows[3, :3] = [4, 4, 7]                                   # norms 3, 7, 9, 9
    x = enc(np.round(rng.standard_normal((M, K)) * 4) / 4)
    b = enc(np.round(rng.standard_normal(4) * 8) / 8) if with_bias else None
    down = enc(np.round(rng.standard_normal((2, K)) * 4) / 4)
    return x, enc(rows), b, down, enc(np.zeros((4, 2)))


@pytest.mark.parametrize("dt", [F16, BF16, F32])
def test_dora_unit_gain_is_the_lora_forward(dt):
    """With up = 0 the merged weight is W; a magnitude equal to each row's norm
    gives gain 1, so y is the LoRA forward (bias added unscaled); a magnitude
    of twice the norm gives the forward of 2W."""
    rng = np.random.default_rng(31)
    x, w, b, down, up = _dora_case(dt, rng)
    m1 = oracle.encode(np.array([3.0, 7.0, 9.0, 9.0]), dt)
    got = oracle.dora_forward(x, dt, w, dt, b, dt, down, dt, up, dt, m1, dt, scale=1.5)
    lora = oracle.forward(x, dt, w, dt, b, dt, down, dt, up, dt, scale=1.5)
    np.testing.assert_array_equal(got["y"], lora["y"])
    assert got["norms"].tolist() == [3.0, 7.0, 9.0, 9.0]
    m2 = oracle.encode(np.array([6.0, 14.0, 18.0, 18.0]), dt)
    w2 = oracle.encode(2 * oracle.as_float64(w, dt).ravel(), dt).reshape(w.shape)
    got2 = oracle.dora_forward(x, dt, w, dt, b, dt, down, dt, up, dt, m2, dt, scale=1.5)
    np.testing.assert_array_equal(got2["y"], oracle.forward(x, dt, w2, dt, b, dt, down, dt, up, dt, scale=1.5)["y"])


def test_dora_is_invariant_to_the_scale_of_the_merged_weight():
    """Doubling W and up doubles the merged weight and its norms: y is unchanged."""
    rng = np.random.default_rng(32)
    dt = BF16
    M, N, K, r = 6, 5, 16, 3
    x, w, d, u = (_draw(rng, s, dt, 0.5) for s in ((M, K), (N, K), (r, K), (N, r)))
    b, mag = _draw(rng, (N,), dt, 0.5), _draw(rng, (N,), dt)
    dbl = lambda a: oracle.encode(2 * oracle.as_float64(a, dt).ravel(), dt).reshape(a.shape)
    y1 = oracle.dora_forward(x, dt, w, dt, b, dt, d, dt, u, dt, mag, dt, scale=0.75)
    y2 = oracle.dora_forward(x, dt, dbl(w), dt, b, dt, d, dt, dbl(u), dt, mag, dt, scale=0.75)
    np.testing.assert_array_equal(y1["y"], y2["y"])
    np.testing.assert_array_equal(y2["norms"], 2 * y1["norms"])
    # a row subset is the same rows of the full evaluation
    part = oracle.dora_forward(x, dt, w, dt, b, dt, d, dt, u, dt, mag, dt, scale=0.75, rows=[4, 1])
    np.testing.assert_array_equal(part["y"], y1["y"][[4, 1]])


def test_dora_policy():
    rng = np.random.default_rng(33)
    x, w, d, u = (_draw(rng, s, F16) for s in ((2, 8), (3, 8), (1, 8), (3, 1)))
    got = oracle.dora_forward(x, F16, w, F16, None, None, d, F16, u, F16, _draw(rng, (3,), F32), F32)
    assert got["compute"] == F16 and got["output"] == F32             # an fp32 magnitude promotes y
    with pytest.raises(oracle.OracleError):
        oracle.dora_forward(x, F16, w, F16, None, None, d, F16, u, F16, _draw(rng, (3,), BF16), BF16)
