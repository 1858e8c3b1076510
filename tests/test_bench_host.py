"""Host logic of bench.py, on the CPU: which step a kernel's counters belong
to, the per-call HBM figures the counter summary derives from rocprofv3's
per-dispatch values, the source digest that keeps a summary tied to the code
it was taken from, and the warmup rule."""
import csv
import importlib.util
import os
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_kernel_step_reads_the_kernel_family(bench):
    ks = bench.kernel_step
    # rocprofv3 prints full signatures; a template argument spelled "true"
    # (the gather flag of the matrix-core expand) must not change the step
    assert ks("void lora::(anonymous namespace)::k_expand_mfma<4, true, 4>"
              "(lora::LaneGeom, lora::PoolDev, lora::RoutingDev, int)") == "expand"
    assert ks("k_expand_mfma<2, false, 4>") == "expand"
    assert ks("k_shrink_mfma<false, 2, 2, true>") == "shrink"
    assert ks("k_shrink_gemv<true, 4, true>") == "shrink"
    assert ks("k_expand_gemv<2, 4>") == "expand"
    assert ks("k_delta_gemv<false>") == "delta"
    for other in ("k_linear<128, 128, true>", "k_route_decode<512, 4, true>",
                  "__amd_rocclr_copyBuffer", "k_pack_a", "k_set_meta",
                  "Cijk_Alik_Bljk_BSS_BH_Bias_S_HA_S_SAV_UserArgs_MT256x256x64_"):
        assert ks(other) == "", other


def _write_run(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Value": value})


def test_summarize_pmc_counts_each_dispatch_once(bench, tmp_path, monkeypatch):
    """A mixed batch (tp_share: two lanes, GEMV and matrix-core kernels of
    both steps) with known per-dispatch KiB: every kernel is counted once per
    call, in its own step, and scaled by the copy calibration."""
    pmc = tmp_path / "pmc"
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_digest", lambda: "digest-under-test")
    calls = (bench.PMC_STEPS + bench.PMC_WARMUP) * bench.PMC_LAYERS * 2
    per_call = {  # kernel: (FETCH KiB, WRITE KiB) per dispatch, one dispatch a call
        "k_shrink_gemv<true, 4, true>(lora::LaneGeom)": (10.0, 1.0),
        "k_shrink_mfma<false, 2, 2, true>(lora::LaneGeom)": (20.0, 2.0),
        "k_expand_gemv<4, 8>(lora::LaneGeom)": (30.0, 40.0),
        "k_expand_mfma<4, true, 4>(lora::LaneGeom)": (50.0, 60.0),
    }
    others = [("k_pack_a(unsigned short*)", 999.0), ("k_route_decode<64, 4, false>", 7.0)]
    for n, i in (("fetch", 0), ("write", 1)):
        _write_run(str(pmc / f"tp_share_{n}"),
                   [(k, v[i]) for k, v in per_call.items() for _ in range(calls)] + others)
    # a 256 MiB copy that FETCH_SIZE reads as half its bytes, WRITE_SIZE as all
    copy = bench.COPY_CALIBRATION_BYTES / 1024
    _write_run(str(pmc / "copy_fetch"), [("__amd_rocclr_copyBuffer", copy / 2)] * 3)
    _write_run(str(pmc / "copy_write"), [("__amd_rocclr_copyBuffer", copy)] * 3)
    bench.summarize_pmc(str(pmc), ["tp_share"])
    import json
    doc = json.load(open(tmp_path / "profiles" / "traffic.json"))["tp_share"]
    want = {"shrink": (30.0, 3.0), "expand": (80.0, 100.0), "delta_apply": (110.0, 103.0)}
    for part, (f_kib, w_kib) in want.items():
        rec = doc[part]
        assert rec["calls"] == calls
        assert rec["fetch_kib_per_call"] == pytest.approx(f_kib)
        assert rec["write_kib_per_call"] == pytest.approx(w_kib)
        assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
        assert rec["hbm_bytes_per_call"] == int(f_kib * 1024 * 2 + w_kib * 1024)
        assert rec["sources_sha256"] == "digest-under-test"
    assert doc["expand"]["kernels"] == ["k_expand_gemv", "k_expand_mfma"]
    assert bench.recorded_traffic("tp_share", "expand") == int(80 * 1024 * 2 + 100 * 1024)
    monkeypatch.setattr(bench, "sources_digest", lambda: "other sources")
    assert bench.recorded_traffic("tp_share", "expand") is None


def test_sources_digest_follows_code_not_comments(bench, tmp_path, monkeypatch):
    (tmp_path / "include").mkdir()
    csrc = tmp_path / "adapter_deltas_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "include" / "lora.h").write_text("int f(int a); // entry\n")
    k = csrc / "kernels_x.hip"
    k.write_text("__global__ void k(int *p) { p[0] = 1; }\n")
    lin = csrc / "kernels_linear.hip"
    lin.write_text("__global__ void l(int *p) { p[0] = 2; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.sources_digest()
    k.write_text("// a comment\n__global__ void k(int *p)\n{\n    p[0] = 1;   /* note */\n}\n")
    assert bench.sources_digest() == d0
    lin.write_text("__global__ void l(int *p) { p[0] = 3; }\n")
    assert bench.sources_digest() == d0
    k.write_text("__global__ void k(int *p) { p[0] = 2; }\n")
    assert bench.sources_digest() != d0


def test_warmup_runs_the_given_count_or_a_floor(bench, monkeypatch):
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    n = [0]

    def step():
        n[0] += 1
    args = types.SimpleNamespace(warmup=3)
    bench.warmup(args, step)
    assert n[0] == 3 and args.warmup == 3
    args = types.SimpleNamespace(warmup=0)
    n[0] = 0
    bench.warmup(args, step)
    assert n[0] == 0
    monkeypatch.setattr(bench, "WARMUP_MIN_S", 0.02)
    args = types.SimpleNamespace(warmup=None)
    n[0] = 0
    bench.warmup(args, step)
    assert n[0] >= bench.WARMUP_MIN_STEPS and args.warmup == n[0]
