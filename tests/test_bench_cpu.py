"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic
work model behind the roofline line, and the source hash that keys the
recorded HBM counters."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_stage_work_large_layer():
    T, H, E, k, I = 16384, 7168, 256, 8, 2048
    w = bench.stage_work(T, H, E, k, I, touched=E)
    A = T * k
    bound, ops, unit, peak = w["gate_up"]
    assert (bound, unit, peak) == ("mfma", "TOP/s", bench.PEAK_INT8_OPS)
    assert ops == 2 * A * H * 2 * I
    # the down GEMM writes its fp32 output rows (4*A*H bytes): below the ridge
    # point, it is priced against HBM
    bound, nbytes, unit, _ = w["down"]
    assert bound == "hbm" and unit == "GB/s"
    assert nbytes == E * (H * I + 4 * H) + A * I + 8 * A + 4 * A * H
    assert 2 * A * I * H / nbytes < bench.PEAK_INT8_OPS / bench.PEAK_HBM
    # memory-bound stages are priced in bytes: fp32 in, codes out, one scale per row
    assert w["quant"] == ("hbm", 4 * T * H + T * H + 4 * T, "GB/s", bench.PEAK_HBM)
    assert w["combine"] == ("hbm", 4 * A * H + 4 * T * H, "GB/s", bench.PEAK_HBM)
    # FP8 codes: the same work against the FP8 peak
    # FP8 codes: the same work against the peak of the matrix cores that run it
    # (exact products on the bf16 cores; the fast path on the FP8 cores)
    assert bench.stage_work(T, H, E, k, I, E, "fp8")["gate_up"][2:] == ("TFLOP/s", bench.PEAK_BF16_OPS)
    assert bench.stage_work(T, H, E, k, I, E, "fp8_fast")["gate_up"][2:] == ("TFLOP/s", bench.PEAK_FP8_OPS)


def test_stage_work_decode_layer_is_hbm_bound():
    T, H, E, k, I = 64, 4096, 64, 2, 1536
    w = bench.stage_work(T, H, E, k, I, touched=51)
    bound, nbytes, unit, _ = w["gate_up"]
    assert bound == "hbm" and unit == "GB/s"
    # the touched experts' gate-up weights and scales dominate
    assert nbytes >= 51 * 2 * I * H


def test_source_hash_ignores_comments_only():
    a = "int f() { return 1; } // one\n/* block\n comment */\nint g;\n"
    b = "int f() { return 1; }\n\n\nint g;   \n"
    c = "int f() { return 2; }\nint g;\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_counter_fields_scale_to_the_sustained_clock():
    ent = {"fetch_bytes": 1000, "write_bytes": 24, "clock_mhz": 1800.0, "mfma_busy": 0.6}
    f = bench.counter_fields(ent, "mfma", achieved=2.0e15, peak=5.0e15)
    assert f["traffic"] == 1024
    assert f["sustained_clock_mhz"] == 1800.0
    # 2.0 of 5.0 POP/s at 2400 MHz is 2.0 of 3.75 at 1800 MHz
    assert abs(f["frac_at_sustained_clock"] - 2.0 / 3.75) < 1e-4
    # memory-bound kernels carry traffic only; no record, no fields
    assert bench.counter_fields(ent, "hbm", 1.0, 2.0) == {"traffic": 1024}
    assert bench.counter_fields(None, "mfma", 1.0, 2.0) == {"traffic": None}


def test_committed_counters_cover_the_dominant_stages():
    with open(bench.COUNTERS_FILE) as f:
        rec = json.load(f)
    st = rec["stages"]
    for key in ("large:gate_up", "large:down", "prefill:gate_up", "decode:gate_up", "dense:gemm",
                "large/fp8:gate_up"):
        assert key in st, key
        assert st[key]["fetch_bytes"] > 0 and st[key]["avg_us"] > 0
    # the matrix-bound kernels carry the clock they ran at, below the peak clock
    for key in ("large:gate_up", "large:down", "dense:gemm"):
        assert 1000 < st[key]["clock_mhz"] <= bench.PEAK_CLOCK_MHZ
        assert 0 < st[key]["mfma_busy"] < 1
