"""Host logic of bench.py that needs no GPU: the copy/compute overlap read from a trace."""
import csv
import os

import bench


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_interval_algebra():
    u = bench._union([(10, 12), (0, 5), (3, 8)])
    assert u == [[0, 8], [10, 12]] and bench._cover(u) == 10
    assert bench._meet(u, bench._union([(4, 11)])) == 5
    assert bench._meet(u, []) == 0


def test_overlap_of_dma_copies(tmp_path):
    kh = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    # set-up kernel before the first router launch, then two passes of copies and GEMMs
    _write(tmp_path / "run_kernel_trace.csv", kh, [
        ["at::fill", 0, 50],
        ["void moe::router_kernel<...>", 100, 110],
        ["void moe::gu_kernel<...>", 120, 220],       # half under the copy [100, 170)
        ["void moe::down_kernel<...>", 300, 340],     # fully under the copy [290, 400)
        ["void moe::topk_kernel", 500, 510],          # after the last copy: outside the window
    ])
    ch = ["Kind", "Direction", "Start_Timestamp", "End_Timestamp"]
    _write(tmp_path / "run_memory_copy_trace.csv", ch, [
        ["MEMORY_COPY", "MEMORY_COPY_HOST_TO_DEVICE", 20, 60],    # before the router: set-up
        ["MEMORY_COPY", "MEMORY_COPY_HOST_TO_DEVICE", 100, 170],
        ["MEMORY_COPY", "MEMORY_COPY_DEVICE_TO_HOST", 170, 290],  # not host to device
        ["MEMORY_COPY", "MEMORY_COPY_HOST_TO_DEVICE", 290, 400],
    ])
    r = bench.overlap_from_trace(str(tmp_path))
    assert r["copy_kind"] == "dma" and r["copies"] == 2
    assert r["window_ms"] == round(300 / 1e6, 3)
    assert r["link_busy_frac"] == round(180 / 300, 4)
    # GEMMs busy 140 ns, 50 + 40 of them under a copy
    assert r["gemm_under_copy_frac"] == round(90 / 140, 4)
    # all library kernels in the window: router 10 (under), gu 100 (50 under), down 40 (under)
    assert r["kernels_under_copy_frac"] == round(100 / 150, 4)


def test_overlap_prefers_line_copy_kernels(tmp_path):
    kh = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    _write(tmp_path / "a_kernel_trace.csv", kh, [
        ["void moe::router_kernel<...>", 0, 10],
        ["void moe::line_copy_kernel(...)", 10, 110],
        ["void moe::gu_kernel<...>", 50, 150],
        ["void moe::line_copy_kernel(...)", 150, 250],
    ])
    ch = ["Kind", "Direction", "Start_Timestamp", "End_Timestamp"]
    # a later link probe: ignored once the run copies with kernels
    _write(tmp_path / "a_memory_copy_trace.csv", ch,
           [["MEMORY_COPY", "MEMORY_COPY_HOST_TO_DEVICE", 400, 900]])
    r = bench.overlap_from_trace(str(tmp_path))
    assert r["copy_kind"] == "kernel" and r["copies"] == 2
    assert r["link_busy_frac"] == round(200 / 240, 4)
    assert r["gemm_under_copy_frac"] == 0.6
    assert os.path.basename(r["trace"]) == os.path.basename(str(tmp_path))
