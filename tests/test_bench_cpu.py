"""The benchmark's host-side parts on the CPU: its algorithmic-work formulas, the traffic file
lookup and its oracle baselines (the cpu_baseline leg) on tiny workloads of each kind."""
import json
import math

import pytest

import bench
from kv_cache_quantization_tile_amd import synth


def test_flop_formula_and_peaks():
    # 7 butterfly stages of 16384 add/sub, 4 x 16384 FMA per iteration, ~131072 for RTN
    assert bench.quant_flop_per_tile(0) == 7 * 16384 + 131072
    assert bench.quant_flop_per_tile(8) - bench.quant_flop_per_tile(7) == 131072
    # 256 CU x 4 SIMD x 64 lanes x 2 FLOP every 2 cycles at 2.4 GHz
    assert math.isclose(bench.FP32_VECTOR_PEAK_TFLOPS, 256 * 4 * 64 * 2 / 2 * 2.4e9 / 1e12, rel_tol=1e-3)


def test_traffic_lookup(tmp_path, monkeypatch):
    """bench reads measured bytes per launch only for the sources they were measured on."""
    t = json.load(open(bench.os.path.join(bench.ROOT, "profiles", "traffic.json")))
    src = t["source_hash"]
    k = t["workloads"]["one_layer_16k"]["kernels"]["quantize_kv_kernel"]["bytes_per_launch"]
    assert bench.load_traffic("quantize_kv_kernel", src, "one_layer_16k") == k
    assert bench.load_traffic("quantize_kv_kernel", "0" * 16, "one_layer_16k") is None
    assert bench.load_traffic("no_such_kernel", src, "one_layer_16k") is None


def test_cpu_baseline_quantize_and_decode():
    w = synth.one_layer(device="cpu", context=1024)
    t_step, cores, sample = bench.cpu_baseline(w, 2, budget_s=0.5)
    assert t_step > 0 and cores >= 1 and "tiles quantized" in sample


@pytest.mark.parametrize("maker", [
    lambda: synth.batched_paged(device="cpu", batch=3, lo=256, hi=700, steps=2),
    lambda: synth.long_context(device="cpu", context=1024, steps=2),
])
def test_cpu_baseline_decode(maker):
    w = maker()
    t_step, cores, sample = bench.cpu_baseline_decode(w, 2, budget_s=0.5, tail=3)
    assert t_step > 0 and cores >= 1 and "pages" in sample


def _write_counters(d, rows):
    import csv as _csv
    import os as _os
    _os.makedirs(d, exist_ok=True)
    with open(_os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = _csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i, k, c, v])


def test_reduce_profiles(tmp_path):
    """The profile reduction on a fake rocprofv3 tree: traffic scaled by the calibration copy,
    SQ counters per wave, issue share from GRBM cycles."""
    import os as _os
    d = tmp_path / "prof"
    qk = "void kvarn::(anonymous namespace)::quantize_kv_kernel<4, 2>(__half const*)"
    dk = "void kvarn::(anonymous namespace)::decode_pages_kernel<4, 2, 2, true>(__half const*)"
    copy = "__amd_rocclr_copyBuffer"
    mib = bench.CALIB_MB * 1024
    _os.makedirs(d / "t_prefill_burst", exist_ok=True)
    with open(d / "t_prefill_burst" / "run_kernel_stats.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write(f'"{qk}",2,8000000,4000000.0,90,3900000,4100000,1\n')
        f.write(f'"{dk}",2,320000,160000.0,5,150000,170000,1\n')
    # copy reads half of its bytes through FETCH_SIZE (factor 2), writes all
    _write_counters(d / "f_prefill_burst", [(qk, "FETCH_SIZE", 1000.0), (qk, "FETCH_SIZE", 1200.0),
                                            (copy, "FETCH_SIZE", mib / 2)])
    _write_counters(d / "w_prefill_burst", [(qk, "WRITE_SIZE", 300.0), (copy, "WRITE_SIZE", mib)])
    i_rows, a_rows = [], []
    for k, valu in ((qk, 4000.0 * 100), (dk, 900.0 * 10)):
        waves = 100.0 if k == qk else 10.0
        i_rows += [(k, "SQ_INSTS_VALU", valu), (k, "SQ_INSTS_MFMA", 64 * waves),
                   (k, "SQ_INSTS_LDS", 10 * waves), (k, "SQ_INSTS_SALU", waves),
                   (k, "SQ_INSTS_VMEM_RD", waves), (k, "SQ_INSTS_VMEM_WR", waves),
                   (k, "SQ_WAVES", waves), (k, "SQ_BUSY_CYCLES", 1.0),
                   (k, "GRBM_GUI_ACTIVE", 8 * 1000.0)]
        a_rows += [(k, "SQ_ACTIVE_INST_VALU", valu), (k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 100.0),
                   (k, "SQ_ACTIVE_INST_LDS", 100.0), (k, "SQ_LDS_BANK_CONFLICT", 40.0),
                   (k, "SQ_WAVE_CYCLES", 1.0), (k, "SQ_WAIT_INST_ANY", 1.0),
                   (k, "SQ_ACTIVE_INST_ANY", 1.0), (k, "SQ_BUSY_CU_CYCLES", 1.0),
                   (k, "GRBM_GUI_ACTIVE", 8 * 1000.0)]
    _write_counters(d / "i_prefill_burst", i_rows)
    _write_counters(d / "a_prefill_burst", a_rows)
    out = tmp_path / "out"
    out.mkdir()
    bench.reduce_profiles(str(d), str(out))
    t = json.load(open(out / "traffic.json"))
    q = t["workloads"]["prefill_burst"]["kernels"]["quantize_kv_kernel"]
    assert t["workloads"]["prefill_burst"]["calibration"]["fetch_factor"] == 2.0
    assert q["read_bytes"] == int(1100.0 * 1024 * 2) and q["write_bytes"] == int(300.0 * 1024)
    c = json.load(open(out / "counters.json"))["workloads"]["prefill_burst"]
    assert c["quantize_kv_kernel"]["valu_per_wave"] == 4000.0
    assert c["quantize_kv_kernel"]["mfma_per_wave"] == 64.0
    # 400000 VALU x 2 cycles over 1024 SIMDs x 1000 cycles
    assert math.isclose(c["quantize_kv_kernel"]["valu_issue"], round(400000 * 2 / 1024e3, 4))
    assert math.isclose(c["quantize_kv_kernel"]["mfma_busy"], 0.1)
    assert math.isclose(c["quantize_kv_kernel"]["lds_conflict"], 0.1)
    txt = open(out / (bench.PROFILE_FILES["prefill_burst"] + ".txt")).read()
    assert "quantize_kv_kernel" in txt and "rocprofv3 --pmc FETCH_SIZE" in txt


def test_percentiles():
    p = bench.percentiles([1.0, 2.0, 3.0, 4.0, 5.0])
    assert p["p50"] == 3.0 and p["mean"] == 3.0 and p["n"] == 5
    assert math.isclose(p["p10"], 1.4) and math.isclose(p["p90"], 4.6)
