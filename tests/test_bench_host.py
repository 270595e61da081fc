"""Host logic of the measurement, no GPU: bench.py's refusal of more than one GPU,
the algorithmic work its rates divide by, and the HBM-traffic record it reads
(keyed by a hash of the library sources)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from mixture_experts_ffn_int32_amd.roofline import (PEAK_BF16_TFLOPS, PEAK_FP8_TFLOPS,  # noqa: E402
                                                    PEAK_HBM_GBS, stage_work)

PRODUCTS = ("gmm1_swiglu", "gmm2", "act_grad", "input_grad", "dw1", "dw2")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_products_count_18_shi_flops():
    # per routed row: up-projection 4HI, down-projection 2HI (forward 6HI); act_grad
    # 2HI, input_grad 4HI, W2Grad 2HI, W1Grad 4HI (backward 12HI)
    T, H, I, E, K = 8192, 7168, 2048, 32, 8
    S = T * K
    work = {s: stage_work(s, T, H, I, E, K) for s in PRODUCTS}
    assert all(w[0] == "mfma" and w[3] == PEAK_BF16_TFLOPS for w in work.values())
    assert sum(w[1] for w in work.values()) == 18 * S * H * I
    assert work["gmm1_swiglu"][1] + work["gmm2"][1] == 6 * S * H * I
    # small problems pair two products in one launch: both count
    for pair, a, b in (("act_grad+dw2", "act_grad", "dw2"), ("input_grad+dw1", "input_grad", "dw1")):
        assert stage_work(pair, T, H, I, E, K)[1] == work[a][1] + work[b][1]
    # small problems route inside the up-projection's launch: the launch does its products
    assert stage_work("route+gmm1_swiglu", T, H, I, E, K) == work["gmm1_swiglu"]
    # the FP8 products take the FP8 peak, with the same flop counts
    assert stage_work("gmm1_fp8_swiglu", T, H, I, E, K)[1:] == (4 * S * H * I, "TFLOP/s", PEAK_FP8_TFLOPS)
    assert stage_work("input_grad_fp8", T, H, I, E, K)[1] == work["input_grad"][1]


def test_shared_expert_adds_its_rows():
    # a shared expert of width Is is one more group of T rows in every product
    T, H, I, E, K, Is = 1024, 512, 128, 4, 2, 256
    for s in PRODUCTS:
        base = stage_work(s, T, H, I, E, K)[1]
        assert stage_work(s + "+shared", T, H, I, E, K, Is=Is)[1] == base + base * T * Is // (T * K * I)


def test_memory_bound_stages_count_each_operand_once():
    T, H, I, E, K = 4000, 2048, 768, 128, 8
    S = T * K
    assert stage_work("route", T, H, I, E, K) == ("hbm", 12 * S, "GB/s", PEAK_HBM_GBS)
    # K gathered bf16 rows, a row index and a weight per slot in; one bf16 row per token out
    assert stage_work("combine", T, H, I, E, K)[1] == S * H * 2 + S * 8 + T * H * 2
    assert stage_work("combine", T, H, I, E, K, f32=True)[1] == S * H * 4 + S * 8 + T * H * 4
    # the weight quantiser: bf16 in, one code byte per element and a float descale per column out
    assert stage_work("quant_w1", T, H, I, E, K)[1] == E * H * 2 * I * 3 + E * 2 * I * 4
    assert stage_work("no_such_stage", T, H, I, E, K) == (None, 0, None, None)


def test_recorded_traffic_is_used_only_for_the_recorded_sources(tmp_path, monkeypatch):
    import bench
    (tmp_path / "profiles").mkdir()
    rec = {"source_sha": "0123456789abcdef",
           "per_workload": {"hotspot": {"dw1": {"fetch_kib": 1.0, "write_kib": 1.0, "bytes": 12126345678.4}}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda: "0123456789abcdef")
    assert bench.recorded_traffic("hotspot", "dw1") == 12126345678
    assert bench.recorded_traffic("hotspot", "gmm2") is None       # no record for that kernel
    assert bench.recorded_traffic("skewed", "dw1") is None         # nor for that workload
    monkeypatch.setattr(bench, "source_sha", lambda: "fedcba9876543210")
    assert bench.recorded_traffic("hotspot", "dw1") is None        # the sources changed since


def test_committed_traffic_record_names_every_workload_of_the_profiles():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        rec = json.load(fh)
    names = sorted(f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.startswith("step_kernels_"))
    workloads = sorted(f[len("step_kernels_"):].split("_")[0] for f in names)
    assert sorted(rec["per_workload"]) == workloads
    for wl, kernels in rec["per_workload"].items():
        assert kernels and all(v["bytes"] >= 0 for v in kernels.values()), wl
