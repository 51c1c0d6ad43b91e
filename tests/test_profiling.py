"""The profile summarisers (persistent_stream_tiling_amd.profiling) on small
synthetic rocprofv3 outputs whose answers are known: which dispatches count
as timed steps, the traffic calibration against the plain copy, counter
means, the derived L2 figures, the repack share and the operand-value table."""
import csv
import json
import os

import pytest

from persistent_stream_tiling_amd import profiling

GEMM = "void gsk::gemm_kernel_pp<1>(gsk::KernelArgs)"
FILL = "void at::native::vectorized_elementwise_kernel<16>(int)"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _trace(dirname, durations_us):
    """A kernel trace: a cache fill before every GEMM dispatch."""
    rows, t = [], 1000
    for d in durations_us:
        rows.append(dict(Kernel_Name=FILL, Start_Timestamp=t, End_Timestamp=t + 500))
        t += 1000
        rows.append(dict(Kernel_Name=GEMM, Start_Timestamp=t, End_Timestamp=t + int(d * 1000)))
        t += int(d * 1000) + 1000
    _write(os.path.join(dirname, "run_kernel_trace.csv"), rows)


def _counters(dirname, dispatches):
    """Counter rows: dispatches is a list of (kernel, us, {counter: value})."""
    rows, t = [], 0
    for i, (name, us, vals) in enumerate(dispatches):
        for k, v in vals.items():
            # two rows per counter (dies / channels), summed by the reader
            for part in (0.25, 0.75):
                rows.append(dict(Kernel_Name=name, Dispatch_Id=i, Start_Timestamp=t,
                                 End_Timestamp=t + int(us * 1000), Counter_Name=k,
                                 Counter_Value=v * part))
        t += int(us * 1000) + 1000
    _write(os.path.join(dirname, "run_counter_collection.csv"), rows)


def test_trace_counts_only_the_timed_gemm_launches(tmp_path):
    # two schedules of 2 warm-up + 3 timed launches; warm-ups are slow
    _trace(str(tmp_path), [50, 50, 10, 12, 14, 60, 60, 20, 20, 20])
    text, means = profiling.trace_summary(str(tmp_path), ["dp", "hybrid"], 2, 3, "cmd")
    assert means == pytest.approx({"dp": 12.0, "hybrid": 20.0})
    assert "gsk::gemm_kernel_pp<1>" in text and "| dp |" in text


def test_trace_beside_the_bench_events(tmp_path):
    line = dict(value=2.0, unit="TFLOP/s", ms_per_step=0.03, config=dict(M=2, N=3, K=5, schedule="dp"),
                roofline=dict(frac=0.5, traffic=None), schedules=dict(dp=dict(ms=0.015)))
    log = tmp_path / "b.log"
    log.write_text("[bench] noise\n" + json.dumps(line) + "\n")
    assert profiling.bench_line(str(log))["value"] == 2.0
    text = profiling.trace_vs_events({"dp": 12.0}, line)
    # events 15 us over a 12 us kernel: 1.25
    assert "| dp | 12.00 | 15.00 | 1.250 |" in text


def test_traffic_is_calibrated_against_the_copy(tmp_path):
    copy_kib = (256 << 20) / 1024.0
    # FETCH reads the copy twice over (factor 0.5), WRITE once (factor 1)
    _counters(str(tmp_path / "f"), [("__amd_rocclr_copyBuffer", 50, {"FETCH_SIZE": 2 * copy_kib})] +
              [(GEMM, 100, {"FETCH_SIZE": 4000.0})] * 3)
    _counters(str(tmp_path / "w"), [("__amd_rocclr_copyBuffer", 50, {"WRITE_SIZE": copy_kib})] +
              [(GEMM, 100, {"WRITE_SIZE": 1000.0})] * 3)
    r = profiling.traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    assert r["fetch"]["factor"] == pytest.approx(0.5)
    assert r["fetch"]["gemm_bytes"] == pytest.approx(4000.0 * 1024 * 0.5)
    assert r["write"]["gemm_bytes"] == pytest.approx(1000.0 * 1024)


def test_pmc_means_skip_warmups_and_sum_parts(tmp_path):
    d = str(tmp_path)
    _counters(d, [(GEMM, 10, {"TCC_HIT_sum": 100.0, "TCC_MISS_sum": 0.0}),
                  (FILL, 5, {"TCC_HIT_sum": 7.0, "TCC_MISS_sum": 7.0}),
                  (GEMM, 20, {"TCC_HIT_sum": 30.0, "TCC_MISS_sum": 10.0}),
                  (GEMM, 30, {"TCC_HIT_sum": 50.0, "TCC_MISS_sum": 30.0})])
    s = profiling.pmc_summary(d, ["dp"], 1, 2)["dp"]
    assert s["us"] == pytest.approx(25.0)
    assert s["TCC_HIT_sum"] == pytest.approx(40.0) and s["TCC_MISS_sum"] == pytest.approx(20.0)
    text = profiling.pmc_table([d], ["a"], ["w"], ["dp"], 1, 2, "title", ["cmd"])
    assert "66.7%" in text  # 40 / (40 + 20)


def test_l2_derived_figures(tmp_path):
    a, b = str(tmp_path / "a"), str(tmp_path / "b")
    # 100 us, 1.8e5 cycles per die (1.80 GHz), 1e6 requests, 80% hits, 4 sectors each
    _counters(a, [(GEMM, 100, {"TCC_READ_sum": 1e6, "TCC_HIT_sum": 8e5, "TCC_MISS_sum": 2e5,
                               "TCC_BUSY_sum": 0.5 * 128 * 1.8e5, "GRBM_GUI_ACTIVE": 8 * 1.8e5})] * 4)
    _counters(b, [(GEMM, 100, {"TCC_READ_SECTORS_sum": 4e6, "TCC_REQ_sum": 1e6,
                               "GRBM_GUI_ACTIVE": 8 * 1.8e5})] * 4)
    text = profiling.l2_report(a, b)
    assert "clock 1.80 GHz" in text
    assert "| L2 hit rate (TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)) | 80.0% |" in text
    assert "0.128 GB (4.00 sectors = 128 B per request)" in text
    assert "1.28 TB/s" in text  # 1.28e8 B in 100 us
    assert "/ die cycles) | 50% |" in text


def test_pack_share(tmp_path):
    d = str(tmp_path / "pk")
    _write(os.path.join(d, "tr_kernel_stats.csv"), [
        dict(Name="void gsk::pack_pair_kernel<unsigned short>(gsk::PackJob, gsk::PackJob)",
             Calls=4, TotalDurationNs=40000, AverageNs=10000, Percentage=10.0),
        dict(Name=GEMM, Calls=4, TotalDurationNs=360000, AverageNs=90000, Percentage=80.0),
        dict(Name=FILL, Calls=4, TotalDurationNs=40000, AverageNs=10000, Percentage=10.0)])
    text = profiling.pack_share([d], ["bf16_irregular_x"])
    assert "pack 10.0 us + GEMM 90.0 us" in text and "the pack is 10% of a step" in text


def test_operand_power_report():
    from persistent_stream_tiling_amd.probes import operand_power
    med = {"normal": 125.0, "exponents": 105.0, "ones": 100.0, "zeros": 100.0}
    text = operand_power.report("plan", med, 2.0 * 4096 ** 3, "cmd")
    # 137.4 GFLOP in 125 us: 1099.5 TFLOP/s, 43.7% of the peak
    assert "| normal | 125.0 | 1099.5 | 43.7% | 1.000 |" in text
    assert "| zeros | 100.0 | 1374.4 | 54.6% | 0.800 |" in text


def test_operand_power_counters(tmp_path):
    from persistent_stream_tiling_amd.probes import operand_power
    # one warm-up dispatch per set, then 6 rounds of 4 per set; the clock of
    # set k is 2.0 - 0.1 k GHz (GRBM_GUI_ACTIVE summed over 8 dies) and the
    # MFMA busy cycles half of 1024 SIMDs' cycles
    seq = []
    for k in range(4):
        seq.append((GEMM, 100, {"GRBM_GUI_ACTIVE": 1.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1.0}))
    for _ in range(6):
        for k in range(4):
            ghz = 2.0 - 0.1 * k
            cyc = ghz * 1e3 * 100  # one die, 100 us
            seq += [(GEMM, 100, {"GRBM_GUI_ACTIVE": 8 * cyc,
                                 "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * cyc})] * 4
    _counters(str(tmp_path), seq)
    res = operand_power.counters(str(tmp_path))
    assert res["normal"]["clock_ghz"] == pytest.approx(2.0)
    assert res["zeros"]["clock_ghz"] == pytest.approx(1.7)
    assert res["ones"]["mfma_util"] == pytest.approx(0.5)
    text = operand_power.counters_report(res, "cmd")
    assert "| exponents | 100.0 | 1.90 | 50.0% |" in text


def test_int8_powers_of_two():
    import numpy as np
    from persistent_stream_tiling_amd.probes import operand_power
    v = np.array([0, 1, 2, 3, 5, 127, -1, -3, -100, -128], dtype=np.int8)
    assert operand_power.pow2_int8(v).tolist() == [0, 1, 2, 2, 4, 64, -1, -2, -64, -128]


def test_phase_probe_instruments_the_current_kernels():
    # every stamp of the phase probe still finds its place in kernels.hip
    from persistent_stream_tiling_amd import _build
    from persistent_stream_tiling_amd.probes import phases
    src = open(os.path.join(_build.CSRC, "kernels.hip")).read()
    out = phases.instrument(src)
    assert out.count("dbg_stamp(p, 0)") == 2      # ping-pong and ring kernels
    assert out.count("burst_end();") == 2          # both ping-pong groups' bursts
    assert "ps_burst" in out and f"PS_BASE = {phases.PS_BASE}" in out
