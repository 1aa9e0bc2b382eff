"""bench.py's host side, without a GPU: the algorithmic work it divides by,
the roofline side each workload falls on, the HBM-traffic record (parsing,
the copy-probe scaling, the source check), the trace and counter summaries,
and the one-GPU contract."""
import csv
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_work_and_bound_of_each_workload():
    """Bytes = 2MK + KN + 2MN (bf16 X, int8 W, bf16 Y); ops = 4MNK (both
    halves); the ridge is 625 ops per byte."""
    B = _bench()
    from segmented_dual_scale_amd import workloads as W
    expect = {  # name: (bytes, ops, hbm-bound)
        "c1_tiny_outseg": (327_680, 50_331_648, True),
        "c2_adanorm_gemv": (14_198_784, 113_246_208, True),
        "c3_dit_ffn_fc2": (72_351_744, 154_618_822_656, False),
        "c4_attn_out_inseg": (29_571_072, 41_797_287_936, False),
        "c5_flux_ffn_fc2": (320_864_256, 1_391_569_403_904, False),
    }
    for name, (nbytes, ops, hbm) in expect.items():
        wl = W.WORKLOADS[name]
        assert B.alg_bytes(wl) == nbytes, name
        assert B.alg_ops(wl) == ops, name
        assert B.hbm_bound(wl) == hbm, name


def test_traffic_record_scaling_and_source_check(tmp_path, monkeypatch):
    """Counter KiB are scaled by what the same counter reads for the copy
    probe; a record of another kernel source or mode reads as absent."""
    B = _bench()
    monkeypatch.setattr(B, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    kernel, wl = "gemm_tile_kernel", "c3_dit_ffn_fc2"
    rec = (f"kernel: {kernel}\nworkload: {wl}\nmode: bf16\n"
           f"source_sha256: {B.source_digest(kernel)}\n"
           "fetch_kib_per_dispatch: 100.0\nwrite_kib_per_dispatch: 30.0\ndispatches: 8 8\n"
           "copy_bytes: 1048576\ncopy_fetch_kib: 512.0\ncopy_write_kib: 1024.0\n")
    path = tmp_path / "profiles" / f"traffic_{kernel}_{wl}.txt"
    path.write_text("# header line: ignored\n" + rec)
    t = B.read_traffic(kernel, wl, "bf16")
    assert t["copy_scale_fetch"] == pytest.approx(0.5)
    assert t["copy_scale_write"] == pytest.approx(1.0)
    assert t["fetch_bytes"] == pytest.approx(100.0 * 1024 / 0.5)
    assert t["write_bytes"] == pytest.approx(30.0 * 1024)
    assert t["bytes_per_launch"] == pytest.approx(t["fetch_bytes"] + t["write_bytes"])
    assert B.read_traffic(kernel, wl, "signed") is None
    path.write_text(rec.replace(B.source_digest(kernel), "0" * 64))
    assert B.read_traffic(kernel, wl, "bf16") is None


def test_summaries_of_trace_and_counter_csv(tmp_path, capsys):
    B = _bench()
    tdir = tmp_path / "trace"
    tdir.mkdir()
    with open(tdir / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, d in enumerate([1000, 2000, 3000, 4000, 5000]):
            w.writerow(["kern_a", 10_000 * i, 10_000 * i + d])
        w.writerow(["kern_b", 0, 500])
    B.summarize_trace(str(tdir))
    out = capsys.readouterr().out.splitlines()
    row = next(ln for ln in out if ln.rstrip().endswith("kern_a")).split()
    assert row[0] == "5" and float(row[1]) == pytest.approx(3.0) and float(row[3]) == pytest.approx(3.0)
    pdir = tmp_path / "pmc"
    pdir.mkdir()
    with open(pdir / "pmc_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, (a, b) in enumerate([(10, 1), (30, 3)]):
            # a counter split over two rows of one dispatch is summed
            w.writerow([d, "gemm_x", "SQ_WAVES", a / 2])
            w.writerow([d, "gemm_x", "SQ_WAVES", a / 2])
            w.writerow([d, "gemm_x", "SQ_INSTS_MFMA", b])
            w.writerow([d, "other_kernel", "SQ_WAVES", 99])
    B.summarize_pmc([str(pdir)])
    out = capsys.readouterr().out
    assert "other_kernel" not in out
    waves = next(ln for ln in out.splitlines() if "SQ_WAVES" in ln).split()
    assert float(waves[1]) == pytest.approx(20.0) and "(2 dispatches)" in out


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_trace_record_written_and_read_back(tmp_path, monkeypatch, capsys):
    """--ingest-trace keeps only the layer kernel's dispatches; the bench reads
    the record back only for the current kernel source and mode."""
    B = _bench()
    monkeypatch.setattr(B, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    tdir = tmp_path / "trace"
    tdir.mkdir()
    kernel, wl = "gemm_smallm_kernel", "c2_adanorm_gemv"
    with open(tdir / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        # five warm-up dispatches of 50 us, then the timed ten of 1..10 us
        for i in range(5):
            w.writerow([f"void sq::{kernel}<1>(args)", 1000 * i, 1000 * i + 50_000])
        for i in range(10):
            t0 = 10_000_000 + 100_000 * i
            w.writerow([f"void sq::{kernel}<1>(args)", t0, t0 + 1000 * (i + 1)])
        w.writerow(["sqprobe_stream_read", 0, 99_000])
    B.ingest_trace(str(tdir), wl, "bf16", kernel, "python3 bench.py --no-all", 10)
    capsys.readouterr()
    t = B.read_trace(kernel, wl, "bf16")
    assert t["calls"] == 10
    assert t["mean_us"] == pytest.approx(5.5)
    assert t["median_us"] == pytest.approx(6.0) and t["p10_us"] == pytest.approx(2.0)
    assert t["p90_us"] == pytest.approx(10.0)
    assert B.read_trace(kernel, wl, "signed") is None
    path = tmp_path / "profiles" / f"trace_{kernel}_{wl}.txt"
    path.write_text(path.read_text().replace(B.source_digest(kernel), "0" * 64))
    assert B.read_trace(kernel, wl, "bf16") is None


def test_kernel_named_for_each_workload_and_mode():
    """The roofline and profile records name the kernel that runs the GEMM
    launch: the LDS-staged kernel for c5 (four K-segments of 3072, codes
    from the quantise-first launch or the caller), the tile kernel for one
    segment or 64-wide head segments, the streaming kernel at small M."""
    B = _bench()
    import segmented_dual_scale_amd as S
    from segmented_dual_scale_amd import workloads as W
    expect = {
        ("c1_tiny_outseg", "bf16"): "gemm_tile_kernel",
        ("c2_adanorm_gemv", "bf16"): "gemm_smallm_kernel",
        ("c2_adanorm_gemv", "w4"): "gemm_smallm_kernel",
        ("c3_dit_ffn_fc2", "bf16"): "gemm_tile_kernel",
        ("c3_dit_ffn_fc2", "signed"): "gemm_tile_kernel",
        ("c3_dit_ffn_fc2", "w4"): "gemm_tile_kernel",
        ("c4_attn_out_inseg", "bf16"): "gemm_tile_kernel",
        ("c5_flux_ffn_fc2", "bf16"): "gemm_lds_kernel",
        ("c5_flux_ffn_fc2", "signed"): "gemm_lds_kernel",
        ("c5_flux_ffn_fc2", "planes"): "gemm_lds_kernel",
        ("c5_flux_ffn_fc2", "single"): "gemm_lds_kernel",
        ("c5_flux_ffn_fc2", "w4"): "gemm_lds_kernel",
    }
    for (name, mode), kernel in expect.items():
        assert B.workload_kernel(S, W.WORKLOADS[name], mode) == kernel, (name, mode)
    # fused bf16 input beyond the running-sum bound takes the LDS kernel too
    assert B.gemm_kernel_name(64, 2 * 66112, [66112, 66112], False, False) == "gemm_lds_kernel"
    assert B.gemm_kernel_name(64, 2 * 3072, [3072, 3072], False, False) == "gemm_tile_kernel"
    assert B.gemm_kernel_name(64, 128, [64, 64], True, False) == "gemm_tile_kernel"


def test_shader_clock_from_busy_cycles_over_trace_span(tmp_path, capsys):
    """GRBM_GUI_ACTIVE is summed over the 8 XCDs: per XCD it is the kernel's
    cycles, and those over the traced nanoseconds are GHz."""
    B = _bench()
    with open(tmp_path / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerow([1, "gemm_k", "GRBM_GUI_ACTIVE", 8 * 2300])      # 2300 cycles in 1000 ns
        w.writerow([2, "gemm_k", "GRBM_GUI_ACTIVE", 8 * 2100 * 2])  # 4200 cycles in 2000 ns
        w.writerow([3, "gemm_k", "GRBM_GUI_ACTIVE", 8 * 2200])      # 2200 cycles in 1000 ns
        w.writerow([4, "other", "GRBM_GUI_ACTIVE", 5])
    with open(tmp_path / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerow([1, "gemm_k", 0, 1000])
        w.writerow([2, "gemm_k", 5000, 7000])
        w.writerow([3, "gemm_k", 9000, 10000])
        w.writerow([4, "other", 0, 10])
    out = B.summarize_clock(str(tmp_path))
    capsys.readouterr()
    med, lo, hi, n, us = out["gemm_k"]
    assert n == 3 and med == pytest.approx(2.2) and lo == pytest.approx(2.1) and hi == pytest.approx(2.3)
    assert us == pytest.approx(4.0 / 3)
    assert "other" not in out
