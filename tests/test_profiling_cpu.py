"""The rocprofv3 summary writer (host logic): per-launch durations, traffic scaled by the 1 GiB copy's
counters, the H2D streaming summary, and the key: value reader that bench.py uses."""
import argparse
import csv

import pytest

from exact_long_context_cqsa_amd import profiling


def _csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def test_kernel_summary_scales_counters_by_the_copy(tmp_path):
    trace = _csv(tmp_path / "kt.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
                 [["void k_attn<64>(Args)", 100, 1100], ["void k_attn<64>(Args)", 2000, 4000],
                  ["other_kernel", 0, 50]])
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    # the copy of 1 GiB reports half its bytes on FETCH_SIZE (KiB) and all of them on WRITE_SIZE
    fetch = _csv(tmp_path / "f.csv", hdr, [["void k_attn<64>(Args)", 256, "FETCH_SIZE", 1000.0],
                                           ["void k_attn<64>(Args)", 256, "FETCH_SIZE", 3000.0],
                                           ["__amd_rocclr_copyBuffer", 1024, "FETCH_SIZE", 524288.0]])
    write = _csv(tmp_path / "w.csv", hdr, [["void k_attn<64>(Args)", 256, "WRITE_SIZE", 500.0],
                                           ["__amd_rocclr_copyBuffer", 1024, "WRITE_SIZE", 1048576.0]])
    args = argparse.Namespace(name="k_attn_case", kernel="k_attn<", trace=trace, fetch=fetch, write=write,
                              command="rocprofv3 ...", note="a note")
    text = profiling.summarise(args)
    out = tmp_path / "s.md"
    out.write_text(text)
    p = profiling.read_profile(str(out))
    assert p["calls"] == "2" and float(p["avg_ns"]) == 1500.0 and p["min_ns"] == "1000"
    assert float(p["fetch_bytes_per_launch"]) == 2000.0 * 1024 * 2     # mean KiB x 1024 x scale 2
    assert float(p["write_bytes_per_launch"]) == 500.0 * 1024
    assert float(p["traffic_bytes_per_launch"]) == 2000.0 * 2048 + 500.0 * 1024
    assert p["kernel_source_sha256"] == profiling.kernel_source_sha256()
    assert "## Notes" in text and "a note" in text


def test_dispatch_selection_by_grid_and_slice(tmp_path):
    """Several phases launch one kernel: --grid keeps one launch shape, --select a slice of the matching
    dispatches in dispatch order (the trace and the counter files alike)."""
    hdr_t = ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
             "End_Timestamp"]
    rows_t = [[1, "merge_kernel<128>", 4096, 1, 1, 0, 100], [2, "merge_kernel<128>", 4096, 1, 1, 200, 400],
              [3, "merge_kernel<128>", 4096, 1, 1, 500, 1100], [4, "merge_kernel<128>", 512, 1, 1, 2000, 2010]]
    trace = _csv(tmp_path / "kt.csv", hdr_t, list(reversed(rows_t)))
    hdr_c = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    cnt = [[i, "merge_kernel<128>", g, "FETCH_SIZE", float(10 * i)] for i, g in ((1, 4096), (2, 4096), (3, 4096), (4, 512))]
    cnt.append([5, "__amd_rocclr_copyBuffer", 1024, "FETCH_SIZE", 524288.0])
    fetch = _csv(tmp_path / "f.csv", hdr_c, cnt)
    assert profiling.trace_stats(trace, "merge_kernel", grid=4096)["calls"] == 3
    st = profiling.trace_stats(trace, "merge_kernel", grid=4096, select="1:3")
    assert st["calls"] == 2 and st["avg_ns"] == 400 and st["min_ns"] == 200
    assert profiling.trace_stats(trace, "merge_kernel", grid=512)["avg_ns"] == 10
    assert profiling.counter_per_dispatch(fetch, "FETCH_SIZE", "merge_kernel", 4096, "1:3") == (25.0, 524288.0)
    assert profiling.counter_per_dispatch(fetch, "FETCH_SIZE", "merge_kernel", 512) == (40.0, 524288.0)


def test_mfma_counter_summary(tmp_path):
    """Executed MFMA FLOPs per launch against the algorithmic count, utilisation, and the clock from
    GRBM_GUI_ACTIVE (summed over 8 XCDs) over the launch's own duration in the same run."""
    hdr_t = ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
             "End_Timestamp"]
    trace = _csv(tmp_path / "kt.csv", hdr_t, [[1, "void fwd_k<64>()", 256, 1, 1, 0, 1000],
                                              [2, "void fwd_k<64>()", 256, 1, 1, 5000, 7000],
                                              [3, "other", 64, 1, 1, 8000, 8100]])
    hdr_c = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    rows = []
    for d, flop, util, gui in ((1, 3.0e9, 40.0, 8 * 2000.0), (2, 5.0e9, 50.0, 8 * 4000.0)):
        rows += [[d, "void fwd_k<64>()", 256, "MfmaFlopsF16", flop], [d, "void fwd_k<64>()", 256, "MfmaFlopsBF16", 0.0],
                 [d, "void fwd_k<64>()", 256, "MfmaUtil", util], [d, "void fwd_k<64>()", 256, "GRBM_GUI_ACTIVE", gui]]
    rows.append([3, "other", 64, "MfmaFlopsF16", 1e12])
    counters = _csv(tmp_path / "c.csv", hdr_c, rows)
    args = argparse.Namespace(name="fwd_k_counters", kernel="fwd_k<", trace=trace, counters=counters,
                              algorithmic_flop=3.2e9, xcds=8, grid=None, select=None, command="rocprofv3 ...",
                              note="")
    out = tmp_path / "m.md"
    out.write_text(profiling.summarise_mfma(args))
    p = profiling.read_profile(str(out))
    assert p["calls"] == "2" and float(p["avg_ns"]) == 1500.0
    assert float(p["mfma_flop_per_launch"]) == 4.0e9 and float(p["executed_over_algorithmic"]) == 1.25
    assert float(p["mfma_util_pct"]) == 45.0 and float(p["clock_ghz"]) == 2.0


def test_copy_summary(tmp_path):
    hdr = ["Kind", "Direction", "Stream_Id", "Source_Agent_Id", "Destination_Agent_Id", "Correlation_Id",
           "Start_Timestamp", "End_Timestamp"]
    rows = [["MEMORY_COPY", "MEMORY_COPY_DEVICE_TO_DEVICE", 1, "Agent 0", "Agent 1", i, 1000 * i, 1000 * i + 400]
            for i in range(5)]
    rows += [["MEMORY_COPY", "MEMORY_COPY_HOST_TO_DEVICE", 0, "Agent 0", "Agent 1", 9, 0, 7000]]
    trace = _csv(tmp_path / "mc.csv", hdr, rows)
    args = argparse.Namespace(name="h2d_case", copy_trace=trace, h2d_stream=1, h2d_bytes=100_000, link_gbs=60.0,
                              command="rocprofv3 --memory-copy-trace ...", note="")
    text = profiling.summarise_copies(args)
    out = tmp_path / "c.md"
    out.write_text(text)
    p = profiling.read_profile(str(out))
    assert p["h2d_copies"] == "5" and p["h2d_busy_ns"] == "2000"
    assert float(p["h2d_gbs"]) == pytest.approx(50.0) and float(p["h2d_frac_of_link"]) == pytest.approx(0.833, abs=1e-3)
    args.h2d_stream = 3
    with pytest.raises(SystemExit):
        profiling.summarise_copies(args)


def test_wave_state_summary(tmp_path):
    """Wave-state shares, VALUBusy and the matrix-core busy share from two counter passes, each read
    from its run directory (kernel trace + counter collection), over the selected dispatches only."""
    hdr_t = ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp",
             "End_Timestamp"]
    hdr_c = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    k = "void fwd_k<64>()"
    dirs = []
    for i, (counters, scale) in enumerate(((profiling.WAVE_STATE_PASS1, 1.0), (profiling.WAVE_STATE_PASS2, 1.0))):
        d = tmp_path / f"p{i}"
        (d / "host").mkdir(parents=True)
        _csv(d / "host" / "run_kernel_trace.csv", hdr_t, [[1, k, 256, 1, 1, 0, 1000], [2, k, 256, 1, 1, 5000, 6000],
                                                           [3, k, 256, 1, 1, 7000, 8000]])
        vals = {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 360.0, "SQ_WAIT_INST_ANY": 350.0,
                "SQ_ACTIVE_INST_ANY": 290.0, "SQ_ACTIVE_INST_LDS": 50.0, "SQ_BUSY_CYCLES": 10.0,
                "SQ_ACTIVE_INST_VALU": 2 * 256 * 0.5 * 1000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 4 * 2 * 256 * 0.25 * 1000.0,
                "GRBM_GUI_ACTIVE": 8 * 2000.0, "SQ_WAVES": 100.0, "SQ_INSTS_VALU": 1360.0, "SQ_INSTS_MFMA": 160.0,
                "SQ_INSTS_SALU": 300.0, "SQ_INSTS_LDS": 240.0, "SQ_INSTS_VALU_TRANS_F32": 320.0,
                "SQ_ACTIVE_INST_SCA": 5.0, "SQ_WAIT_INST_LDS": 6.0}
        rows = []
        for disp in (1, 2, 3):
            f = 1e6 if disp == 1 else 1.0     # the first (warm-up) dispatch is left out by the slice
            rows += [[disp, k, 256, c, vals[c] * f] for c in counters]
        _csv(d / "host" / "run_counter_collection.csv", hdr_c, rows)
        dirs.append(str(d))
    args = argparse.Namespace(name="fwd_k_waves", kernel="fwd_k<", wave_state=",".join(dirs), cus=256, xcds=8,
                              grid=None, select="1:", command="rocprofv3 ...", note="")
    out = tmp_path / "w.md"
    out.write_text(profiling.summarise_wave_state(args))
    p = profiling.read_profile(str(out))
    assert p["calls"] == "2" and float(p["avg_ns"]) == 1000.0 and float(p["clock_ghz"]) == 2.0
    assert float(p["wave_share_issuing"]) == 0.29 and float(p["wave_share_waiting_on_dependency"]) == 0.36
    assert float(p["valu_busy_pct"]) == 50.0 and float(p["mfma_busy_pct"]) == 25.0
    assert p["valu_insts_per_wave"].startswith("13.6") and float(p["mfma_insts_per_wave"]) == 1.6
