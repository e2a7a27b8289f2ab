"""Host logic of the tile planner and of the tuning table (no GPU): the
shortlist's form, the table file's round trip and its refusal of malformed
input, and the forward's workspace covering every shortlisted K split."""
import json

import pytest

import lora_bypass_linear_amd as L

SHAPES = [(4096, 3072, 3072, 16, L.F16), (16, 3072, 3072, 16, L.F16), (128, 3072, 3072, 16, L.F16),
          (16384, 8192, 8192, 128, L.BF16), (8192, 4096, 4096, 64, L.BF16), (1000, 2500, 136, 32, L.F32),
          (64, 128, 8192, 32, L.F32), (1, 8, 8, 16, L.BF16)]


@pytest.mark.parametrize("shape", SHAPES)
def test_shortlist_form(shape):
    M, N, K, rf, c = shape
    plan = L.gemm_plan(M, N, K, rf, c)
    assert 1 <= len(plan) <= 7
    # first: the pick the forward makes by itself
    assert plan[0][:2] == L.gemm_tile(M, N, c)
    assert len({p[:3] for p in plan}) == len(plan)                 # no candidate twice
    for tn, tm, ks, cost in plan:
        assert (tn, tm) in ({(128, 128), (64, 64)} if c == L.F32 else {(256, 256), (192, 256), (128, 128), (64, 64)})
        assert 1 <= ks <= 8 and cost > 0
        tiles = -(-N // tn) * -(-M // tm)
        assert ks == 1 or tiles < 256                                 # a K split only for few tiles
    costs = [p[3] for p in plan[1:]]
    assert costs == sorted(costs)                                     # the rest by modelled time


def test_workspace_covers_every_shortlisted_split():
    M, N, K, r = 16, 3072, 3072, 16
    ks = max(p[2] for p in L.gemm_plan(M, N, K, 16, L.F16))
    assert ks > 1
    assert L.lora_workspace_size(M, N, K, r, L.F16, L.F16, 0, L.F16, L.F16) >= ks * M * N * 4
    # every split the planner could shortlist, whatever order the device's
    # measured rates give: 8 for the 64 x 64 tiles at this shape
    assert L.lora_workspace_size(M, N, K, r, L.F16, L.F16, 0, L.F16, L.F16) >= 8 * M * N * 4


def test_device_rates_without_a_device():
    """No device: 256 CUs and MI355X's published peaks, not measured."""
    r = L.device_rates()
    assert r == {"cus": 256, "mfma16_flops": 2500e12, "mfma32_flops": 157.3e12, "hbm_bytes_per_s": 8e12,
                 "measured": False}


def test_model_time_follows_the_rates():
    """One round of 256 workgroups of 256 x 256 tiles over 8192 K (128 steps of
    64 k plus two fold steps): 2 * 256 * 256 * 64 flops per step at the
    published per-CU rate, plus the fixed launch term."""
    (tn, tm, ks, cost), = L.gemm_plan(4096, 4096, 8192, 128, L.BF16, max_out=1)
    assert (tn, tm, ks) == (256, 256, 1)
    step_s = 2.0 * 256 * 256 * 64 / (2500e12 / 256)
    assert cost == pytest.approx((130 * step_s + 2e-6) * 1e6, rel=1e-12)


def _table(path, lines):
    path.write_text('{"version": 1, "entries": [\n' + ",\n".join(lines) + "\n]}\n")
    return str(path)


def test_table_round_trip(tmp_path):
    L.tuning_clear()
    entries = ['{"key": "gfx950-256cu|lora_fwd|M4096|N3072|K3072|r16|c1|o1", "tile_n": 192, "tile_m": 256, '
               '"ksplit": 1, "ms": 0.071}',
               '{"key": "gfx950-256cu|lora_fwd|M16|N3072|K3072|r16|c1|o1", "tile_n": 64, "tile_m": 64, '
               '"ksplit": 4, "ms": 0.011}']
    assert L.tuning_load(_table(tmp_path / "a.json", entries)) == 2
    assert L.tuning_count() == 2
    out = L.tuning_save(str(tmp_path / "b.json"))
    doc = json.load(open(out))                                       # the saved table is JSON
    got = {e["key"]: (e["tile_n"], e["tile_m"], e["ksplit"]) for e in doc["entries"]}
    assert got == {"gfx950-256cu|lora_fwd|M4096|N3072|K3072|r16|c1|o1": (192, 256, 1),
                   "gfx950-256cu|lora_fwd|M16|N3072|K3072|r16|c1|o1": (64, 64, 4)}
    L.tuning_clear()
    assert L.tuning_count() == 0
    assert L.tuning_load(out) == 2
    L.tuning_clear()


@pytest.mark.parametrize("bad", ['{"key": "k", "tile_n": 100, "tile_m": 256, "ksplit": 1, "ms": 1}',   # no such tile
                                 '{"key": "k", "tile_n": 64, "tile_m": 64, "ksplit": 9, "ms": 1}',      # split > 8
                                 '{"key": "k", "tile_m": 64, "ksplit": 1}'])                          # field missing
def test_malformed_table_is_refused_whole(tmp_path, bad):
    L.tuning_clear()
    good = '{"key": "g", "tile_n": 64, "tile_m": 64, "ksplit": 1, "ms": 1}'
    with pytest.raises(L.LycError) as e:
        L.tuning_load(_table(tmp_path / "t.json", [good, bad]))
    assert e.value.status == L.ERR_IO
    assert L.tuning_count() == 0


def test_default_path_follows_environment(monkeypatch, tmp_path):
    monkeypatch.setenv("LYC_KERNEL_CACHE_DIR", str(tmp_path / "cache"))
    assert L.tuning_cache_path() == str(tmp_path / "cache" / "tuning.json")
    assert L.tuning_load() == 0                                       # no file yet: nothing, no error
