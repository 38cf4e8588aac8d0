"""CPU tests of the rocprofv3 summary tool behind profiles/ and the bench's
roofline traffic figure: kernel statistics, counter means per dispatch, the
copy-kernel calibration, and the staleness check on the kernel sources."""
import os

import pytest

from structured_rank_matmul_amd import profiling


def _write(path, text):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(text)


def test_kernel_stats_sorted_by_total(tmp_path):
    d = tmp_path / "stats"
    _write(str(d / "run_kernel_stats.csv"),
           '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
           '"small",10,1000,100,1,90,110,1\n'
           '"big",2,9000,4500,9,4000,5000,1\n')
    rows = profiling.kernel_stats(str(d))
    assert [r[0] for r in rows] == ["big", "small"]
    assert rows[0][1:] == (2, 9000.0, 4500.0, 4000.0, 5000.0)


def _counters(path, counter, per_dispatch):
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"']
    for did, (name, vals) in enumerate(per_dispatch):
        for v in vals:  # several dimensions of one dispatch are summed
            lines.append(f'{did},"{name}","{counter}",{v}')
    _write(path, "\n".join(lines) + "\n")


def test_traffic_calibration_and_staleness(tmp_path, monkeypatch):
    fetch, write = tmp_path / "f", tmp_path / "w"
    # the copy kernel of 1 MiB reads 1 MiB and writes 1 MiB, but FETCH_SIZE reports half
    _counters(str(fetch / "run_counter_collection.csv"), "FETCH_SIZE",
              [("copy_kernel", [256, 256]), ("gemm_kernel<out>", [300, 300]), ("gemm_kernel<out>", [400, 400])])
    _counters(str(write / "run_counter_collection.csv"), "WRITE_SIZE",
              [("copy_kernel", [1024]), ("gemm_kernel<out>", [2048]), ("gemm_kernel<out>", [2048])])
    means = profiling.counter_means(str(fetch), "FETCH_SIZE")
    assert means["gemm_kernel<out>"] == (2, 700.0)
    out = tmp_path / "traffic.txt"
    profiling.main(["traffic", str(fetch), str(write), "--kernel", "gemm_kernel", "--copy-kernel", "copy",
                    "--copy-bytes", str(1 << 20), "--command-fetch", "f", "--command-write", "w",
                    "--out", str(out)])
    t = profiling.read_traffic(str(out))
    # fetch: 700 KiB * 2 (scale 1 MiB / 512 KiB); write: 2048 KiB * 1
    assert t == pytest.approx((700 * 2 + 2048) * 1024, rel=1e-6)
    # a different source hash makes the figure stale
    monkeypatch.setattr(profiling, "sources_sha256", lambda sources=(), root="": "0" * 64)
    assert profiling.read_traffic(str(out)) is None
    assert profiling.read_traffic(str(tmp_path / "missing.txt")) is None


def test_counter_table_and_derived_mfma_figures(tmp_path):
    d = tmp_path / "pmc"
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"']
    for did in range(2):
        lines += [f'{did},"gemm_kernel<out>","SQ_VALU_MFMA_BUSY_CYCLES",{512000 + did * 0}',
                  f'{did},"gemm_kernel<out>","GRBM_GUI_ACTIVE",4000',
                  f'{did},"gemm_kernel<out>","SQ_INSTS_VALU_MFMA_MOPS_BF16",1000000']
    _write(str(d / "run_counter_collection.csv"), "\n".join(lines) + "\n")
    s = tmp_path / "stats"
    _write(str(s / "run_kernel_stats.csv"),
           '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
           '"gemm_kernel<out>",2,200000,100000,100,100000,100000,0\n')
    t = profiling.counter_table(str(d))
    assert t["gemm_kernel<out>"]["GRBM_GUI_ACTIVE"] == (2, 4000.0)
    out = tmp_path / "c.txt"
    profiling.main(["counters", str(d), "--command", "x", "--stats-dir", str(s), "--simds", "2048",
                    "--out", str(out)])
    text = open(out).read()
    # 512000 / (4000 / 8 * 1024) = 1.0 with the defaults; with 2048 SIMDs 0.5;
    # 512 * 1e6 flop over 100 us = 5.12 TFLOP/s
    assert "mfma_busy" in text and " 0.5000" in text
    line = [ln for ln in text.splitlines() if ln.strip().startswith("mfma_bf16_tflops")][-1]
    assert float(line.split()[-1]) == pytest.approx(5.12, abs=0.05)
