"""The measured tile pick on the GPU: the tuner's winner is one of the
planner's candidates and is what later forward calls of that shape run; every
shortlisted configuration gives results within the oracle's tolerance (a
tuned pick changes speed, never the contract); the table round-trips through
its file with this device's keys."""
import numpy as np
import pytest
import torch

import lora_bypass_linear_amd as L
import workloads as WL
from tests.gpu_cases import oracle_forward, say, score

pytestmark = pytest.mark.gpu

CASES = [("lora_f16_4096x3072x3072_r16", dict(M=16)), ("lora_f16_4096x3072x3072_r16", dict(M=128, N=1024)),
         ("lora_bf16_16384x8192x8192_r128", dict(M=64, N=512, K=1024)),
         ("sweep_xf32_wf32_2048x1280x5120_r32", dict(M=100, N=640, K=256))]


def _setup(name, dims):
    wl = WL.WORKLOADS[name].resized(**dims)
    inputs = WL.generate(wl)
    d = {k: v.to("cuda:0") for k, v in inputs.items()}
    codes = (wl.M, wl.N, wl.K, wl.r, L.dtype_code(d["x"]), L.dtype_code(d["w"]),
             L.dtype_code(d["b"]) if "b" in d else 0, L.dtype_code(d["down"]), L.dtype_code(d["up"]))
    return wl, inputs, d, codes


def _forward(d, wl):
    y = L.lora_linear(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"))
    torch.cuda.synchronize()
    return y.cpu()


@pytest.mark.parametrize("name,dims", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_tuned_pick_is_a_candidate_and_is_used(name, dims):
    L.tuning_clear()
    wl, inputs, d, codes = _setup(name, dims)
    c_dt = L.resolve_dtypes([c for c in codes[4:] if c])[0]
    plan = L.gemm_plan(wl.M, wl.N, wl.K, L.lora_workspace_layout(*codes)[1], c_dt)
    say("tune", wl.name, dims)
    tn, tm, ks, ms, cand = L.lora_linear_tune(d["x"], d["w"], d["down"], d["up"], wl.scale, d.get("b"))
    print(wl.name, "plan", [p[:3] for p in plan], "measured ms", [round(c, 4) for c in cand], "pick", (tn, tm, ks))
    assert (tn, tm, ks) in [p[:3] for p in plan]
    assert ms == pytest.approx(min(cand)) and all(c > 0 for c in cand)
    assert L.tuning_lookup(*codes) == (tn, tm, ks)
    s = score(_forward(d, wl), oracle_forward(inputs, wl), None, wl.K, wl.r)
    assert s["fail"] == 0, s
    L.tuning_clear()


@pytest.mark.parametrize("name,dims", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_every_candidate_meets_the_oracle(name, dims, tmp_path):
    wl, inputs, d, codes = _setup(name, dims)
    c_dt = L.resolve_dtypes([c for c in codes[4:] if c])[0]
    plan = L.gemm_plan(wl.M, wl.N, wl.K, L.lora_workspace_layout(*codes)[1], c_dt)
    key = L.tuning_key(*codes)
    res = oracle_forward(inputs, wl)
    for tn, tm, ks, _ in plan:
        L.tuning_clear()
        f = tmp_path / f"t_{tn}_{tm}_{ks}.json"
        f.write_text('{"version": 1, "entries": [\n{"key": "%s", "tile_n": %d, "tile_m": %d, "ksplit": %d, '
                     '"ms": 1.0}\n]}\n' % (key, tn, tm, ks))
        assert L.tuning_load(str(f)) == 1 and L.tuning_lookup(*codes) == (tn, tm, ks)
        say("candidate", wl.name, (tn, tm, ks))
        s = score(_forward(d, wl), res, None, wl.K, wl.r)
        print(wl.name, (tn, tm, ks), "fail", s["fail"], "ulp", round(s["ulp_max"], 3))
        assert s["fail"] == 0, ((tn, tm, ks), s)
    L.tuning_clear()


def test_tuning_off_takes_the_first_candidate(monkeypatch):
    L.tuning_clear()
    monkeypatch.setenv("LYC_KERNEL_TUNE", "off")
    wl, inputs, d, codes = _setup("lora_f16_4096x3072x3072_r16", dict(M=16))
    plan = L.gemm_plan(wl.M, wl.N, wl.K, 16, L.F16)
    say("tune off")
    tn, tm, ks, ms, cand = L.lora_linear_tune(d["x"], d["w"], d["down"], d["up"], wl.scale)
    assert (tn, tm, ks) == plan[0][:3] and ms == 0.0
    L.tuning_clear()


def test_table_round_trip_on_the_device(tmp_path):
    L.tuning_clear()
    wl, inputs, d, codes = _setup("lora_f16_4096x3072x3072_r16", dict(M=128, N=1024))
    say("tune + save")
    pick = L.lora_linear_tune(d["x"], d["w"], d["down"], d["up"], wl.scale)[:3]
    path = L.tuning_save(str(tmp_path / "tuning.json"))
    L.tuning_clear()
    assert L.tuning_lookup(*codes) is None
    assert L.tuning_load(path) == 1 and L.tuning_lookup(*codes) == pick
    # the key buckets M: a call of 100 tokens shares the 128-token entry
    assert L.tuning_key(100, *codes[1:]) == L.tuning_key(*codes)
    L.tuning_clear()


def test_planner_takes_the_measured_device_rates():
    """The planner's model counts the device's CUs and, once measured, its own
    MFMA and HBM rates.  A sustained MFMA loop runs below the published peak
    (the clock under load stays under the 2.4 GHz it assumes), a device copy
    below 8 TB/s; the modelled time of a one-round GEMM (256 tiles of
    256 x 256 over 128 + 2 steps of 64 k) is then that of the measured rate."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert L.device_rates()["cus"] == cus
    say("measure device rates")
    r = L.measure_device_rates()
    print(r)
    assert r["measured"] and r["cus"] == cus
    assert 1e12 < r["hbm_bytes_per_s"] < 8e12
    assert 0.5e15 < r["mfma16_flops"] < cus * 2500e12 / 256 * 1.01
    assert 0.03e15 < r["mfma32_flops"] < cus * 157.3e12 / 256 * 1.01
    assert L.device_rates() == r
    (tn, tm, ks, cost), = L.gemm_plan(4096, 4096, 8192, 128, L.BF16, max_out=1)
    assert (tn, tm, ks) == (256, 256, 1)
    step_s = 2.0 * 256 * 256 * 64 / (r["mfma16_flops"] / cus)
    rounds = -(-256 // cus)
    assert cost == pytest.approx((rounds * 130 * step_s + 2e-6) * 1e6, rel=1e-9)
