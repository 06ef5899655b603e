"""The rocprofv3 summarisers on small fixtures in rocprofv3's CSV layout (tests/golden/rocprof/:
the headers of rocprofv3 7.2's output with hand-set values, so every figure below follows from
the numbers in those files)."""
import os
import shutil

import pytest

from long_context_la_amd import profiling

FIX = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rocprof")
FWD = r"k_fwd_bf16<0, false, false, false, 128, false, 64>"


def test_short_names():
    assert profiling.short_name("void la::(anonymous namespace)::k_fwd_bf16<0, false, false, false, 128, false, 64>"
                                "(la::FwdArgs)") == "k_fwd_bf16<0, false, false, false, 128, false, 64>"
    assert profiling.short_name("la::(anonymous namespace)::k_state_init(float*, float const*, long)") == \
        "k_state_init"
    assert profiling.short_name("_ZN2la12_GLOBAL__N_18k_decodeIDF16bLi128ELb0EEEvPKT_S4_S4_PS2_PKfPflNS0_2FuE") == \
        "k_decode"


def test_kernel_trace_table():
    rows = profiling.dispatches(os.path.join(FIX, "stats_full", "run_kernel_trace.csv"))
    assert len(rows) == 26
    fwd = profiling.select(rows, FWD, 256)
    assert [round(d["us"]) for d in fwd] == [2000 + 50 * j for j in range(12)]
    table = {(t["kernel"], t["workgroups"]): t for t in profiling.kernel_table(rows)}
    t = table[("k_fwd_bf16<0, false, false, false, 128, false, 64>", 256)]
    assert t["calls"] == 12 and t["min_us"] == pytest.approx(2000) and t["max_us"] == pytest.approx(2550)
    assert t["avg_us"] == pytest.approx(2275) and t["median_us"] == pytest.approx(2275)
    assert table[("k_state_init", 256)]["calls"] == 12
    total = 100 + 120 + 12 * 5 + sum(2000 + 50 * j for j in range(12))
    assert t["pct"] == pytest.approx(100 * 12 * 2275 / total)


def test_traffic_from_fetch_and_write_sizes():
    c = lambda run: os.path.join(FIX, run, "run_counter_collection.csv")
    t = profiling.traffic(c("fetch_full"), c("write_full"), c("copy_fetch"), c("copy_write"), FWD, 4 << 30, 256)
    assert t["fetch_factor"] == pytest.approx(2.0) and t["write_factor"] == pytest.approx(1.0)
    assert t["fetch_kib"] == 3_100_000 and t["write_kib"] == 2_100_000
    assert t["bytes"] == pytest.approx(3_100_000 * 1024 * 2 + 2_100_000 * 1024)


def test_mfma_utilisation_and_clock():
    m = profiling.mfma_utilisation(os.path.join(FIX, "mfma_full", "run_counter_collection.csv"), FWD, 1024, 8,
                                   tiles_per_simd=2048, workgroups=256)
    assert m["kernel_cycles"] == pytest.approx(5e6)
    assert m["utilisation"] == pytest.approx(1_610_612_736 / (5e6 * 1024))
    assert m["busy_per_mfma"] == pytest.approx(16.0)
    assert m["mfma_per_tile_simd"] == pytest.approx(48.0)
    assert m["cycles_per_tile"] == pytest.approx(5e6 / 2048)
    assert m["clock_ghz"] == pytest.approx(2.0)


def test_peaks_from_agent_info_and_rocminfo():
    p = profiling.agent_peaks(os.path.join(FIX, "mfma_full", "run_agent_info.csv"))
    assert p["cus"] == 256 and p["max_clock_mhz"] == 2400
    assert p["bf16_tflops"] == pytest.approx(256 * 2.4e9 * 4096 / 1e12)
    with open(os.path.join(FIX, "rocminfo.txt")) as f:
        assert profiling.parse_rocminfo(f.read()) == (256, 2400)
    assert profiling.parse_rocminfo("no agents") is None
    assert profiling.device_peaks()["bf16_tflops"] > 2000       # rocminfo here, or the datasheet


def test_summaries_are_written_and_read_back(tmp_path):
    out = tmp_path / "raw"
    shutil.copytree(FIX, out)
    prof = tmp_path / "profiles"
    prof.mkdir()
    written = profiling.summarize_all(str(out), str(prof))
    assert "prefill_full_hbm_traffic.txt" in written and "prefill_full_mfma_util.txt" in written
    assert "kernel_stats_prefill_full_64x131072.txt" in written
    traffic = str(prof / "prefill_full_hbm_traffic.txt")
    assert profiling.current_value(traffic, "traffic_bytes") == pytest.approx(3_100_000 * 2048 + 2_100_000 * 1024)
    assert profiling.current_value(str(prof / "prefill_full_mfma_util.txt"), "mfma_utilisation") == \
        pytest.approx(0.3146, abs=1e-4)
    stats = (prof / "kernel_stats_prefill_full_64x131072.txt").read_text()
    assert "rocprofv3 --kernel-trace --stats" in stats and "average 2450.0 us" in stats   # last 5 launches
    # a profile taken on another kernel source is not reported
    text = open(traffic).read().replace(profiling.source_digest(), "0123456789abcdef")
    open(traffic, "w").write(text)
    assert profiling.current_value(traffic, "traffic_bytes") is None


def test_commands_name_committed_files_only():
    for name in profiling.RUNS:
        cmd = profiling.command(name, "$GRAFT_REPO_ROOT/gpurun_out/prof")
        assert cmd.startswith("rocprofv3 ") and " -- python3 $GRAFT_REPO_ROOT/bench.py" in cmd
        assert "_work" not in cmd
    assert not any("--pmc" in profiling.RUNS[n][0] and ("--kernel-trace" in profiling.RUNS[n][0])
                   for n in profiling.RUNS)


def test_cpu_description():
    d = profiling.cpu_description()
    assert d["logical_cpus"] >= 1 and isinstance(d["model"], str)
