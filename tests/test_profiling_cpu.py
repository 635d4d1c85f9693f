"""Host logic of the rocprofv3 summaries (no GPU): the copy-calibrated HBM traffic that
the bench reports as roofline.traffic, its stored form, and the per-kernel counter tables,
on hand-written counter files whose answers follow by arithmetic."""
import csv
import os

import pytest

from vlm_shared_prefix_amd import profiling as PR

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]


def write_run(path, rows):
    """rows: (dispatch id, kernel name, blocks, counter, value); 256 threads per block."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, k, b, c, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Grid_Size": b * 256, "Workgroup_Size": 256,
                        "Counter_Name": c, "Counter_Value": v})


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path):
    """A copy of CALIB_BYTES that reads back as half its size on FETCH_SIZE and its full size on
    WRITE_SIZE gives scales 0.5 and 1.0; the kernel's readings are divided by them.  Copies
    before the calibration fill and other kernels are ignored."""
    kib = PR.CALIB_BYTES / 1024
    gemm = "void jevk::gemm_bf16w<true, true>(args)"
    fetch = [(1, "__amd_rocclr_copyBuffer", 8, "FETCH_SIZE", 1.0),          # an upload, not the calibration
             (2, gemm, 1184, "FETCH_SIZE", 1000.0), (3, gemm, 1184, "FETCH_SIZE", 3000.0),
             (4, "other_kernel", 8, "FETCH_SIZE", 9e9),
             (5, "at::native::vectorized_elementwise_kernel", 8, "FETCH_SIZE", 0.0),
             (6, "__amd_rocclr_copyBuffer", 8, "FETCH_SIZE", kib / 2)]
    write = [(1, gemm, 1184, "WRITE_SIZE", 100.0), (2, gemm, 1184, "WRITE_SIZE", 300.0),
             (3, "at::native::vectorized_elementwise_kernel", 8, "WRITE_SIZE", 0.0),
             (4, "__amd_rocclr_copyBuffer", 8, "WRITE_SIZE", kib)]
    write_run(tmp_path / "f", fetch)
    write_run(tmp_path / "w", write)
    s = PR.summarize(str(tmp_path / "f"), str(tmp_path / "w"), "gemm_bf16w<true, true>")
    assert s["dispatches"] == [2, 2]
    assert s["fetch_scale"] == pytest.approx(0.5) and s["write_scale"] == pytest.approx(1.0)
    assert s["traffic_bytes_per_launch"] == pytest.approx(2000.0 * 1024 / 0.5 + 200.0 * 1024)
    md = tmp_path / "t.md"
    md.write_text(PR.to_markdown(s, "cmd"))
    t, d = PR.stored_traffic(str(md))
    assert t == pytest.approx(s["traffic_bytes_per_launch"], rel=1e-6) and d == PR.source_digest()


def test_traffic_of_one_launch_shape(tmp_path):
    """With a block count, only the dispatches of that launch shape are averaged (the float16
    SwiGLU runs 1184 blocks in a 1024-row prefill and 444 in a 378-row scoring call)."""
    kib = PR.CALIB_BYTES / 1024
    gemm = "void jevk::gemm_bf16w<true, true>(args)"
    fetch = [(1, gemm, 1184, "FETCH_SIZE", 1000.0), (2, gemm, 444, "FETCH_SIZE", 300.0),
             (3, gemm, 1184, "FETCH_SIZE", 3000.0), (4, gemm, 444, "FETCH_SIZE", 500.0),
             (5, "at::native::vectorized_elementwise_kernel", 8, "FETCH_SIZE", 0.0),
             (6, "__amd_rocclr_copyBuffer", 8, "FETCH_SIZE", kib / 2)]
    write = [(1, gemm, 1184, "WRITE_SIZE", 100.0), (2, gemm, 444, "WRITE_SIZE", 30.0),
             (3, "at::native::vectorized_elementwise_kernel", 8, "WRITE_SIZE", 0.0),
             (4, "__amd_rocclr_copyBuffer", 8, "WRITE_SIZE", kib)]
    write_run(tmp_path / "f", fetch)
    write_run(tmp_path / "w", write)
    big = PR.summarize(str(tmp_path / "f"), str(tmp_path / "w"), "gemm_bf16w<true, true>", 1184)
    small = PR.summarize(str(tmp_path / "f"), str(tmp_path / "w"), "gemm_bf16w<true, true>", 444)
    assert big["dispatches"] == [2, 1] and small["dispatches"] == [2, 1]
    assert big["traffic_bytes_per_launch"] == pytest.approx(2000.0 * 1024 / 0.5 + 100.0 * 1024)
    assert small["traffic_bytes_per_launch"] == pytest.approx(400.0 * 1024 / 0.5 + 30.0 * 1024)
    assert "- launch shape: 444 blocks" in PR.to_markdown(small)
    with pytest.raises(ValueError):
        PR.summarize(str(tmp_path / "f"), str(tmp_path / "w"), "gemm_bf16w<true, true>", 999)


def test_traffic_needs_a_calibration_copy(tmp_path):
    write_run(tmp_path / "f", [(1, "gemm_bf16w<true, true>", 8, "FETCH_SIZE", 1.0)])
    write_run(tmp_path / "w", [(1, "gemm_bf16w<true, true>", 8, "WRITE_SIZE", 1.0)])
    with pytest.raises(ValueError):
        PR.summarize(str(tmp_path / "f"), str(tmp_path / "w"), "gemm_bf16w")


def test_source_digest_is_stable():
    d = PR.source_digest()
    assert len(d) == 16 and d == PR.source_digest()
    assert PR.stored_traffic("/nonexistent/summary.md") is None


def test_mfma_table(tmp_path):
    g = "void jevk::gemm_bf16w<true, false>(args)"
    write_run(tmp_path, [(1, g, 448, "MfmaUtil", 40.0), (1, g, 448, "MfmaFlopsBF16", 2e11),
                         (2, g, 448, "MfmaUtil", 60.0), (2, g, 448, "MfmaFlopsBF16", 1e11),
                         (2, g, 448, "MfmaFlopsF16", 1e11), (3, g, 1184, "MfmaUtil", 30.0)])
    md = PR.mfma_markdown(str(tmp_path), "t")
    assert "| gemm_bf16w<true, false> | 448 | 2 | 50.0 | 200.00 |" in md
    assert "| gemm_bf16w<true, false> | 1184 | 1 | 30.0 | 0.00 |" in md


def test_lds_ta_table(tmp_path):
    """TA busy = TA_TA_BUSY_sum / (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs); conflicts per LDS-active
    cycle; LDS waits per wave cycle."""
    g = "void jevk::gemm_bf16w<true, true>(args)"
    rows = []
    for d in (1, 2):
        rows += [(d, g, 1184, "GRBM_GUI_ACTIVE", 8000.0), (d, g, 1184, "TA_TA_BUSY_sum", 256000.0 * 0.5),
                 (d, g, 1184, "SQ_LDS_IDX_ACTIVE", 400.0), (d, g, 1184, "SQ_LDS_BANK_CONFLICT", 100.0),
                 (d, g, 1184, "SQ_WAVE_CYCLES", 1000.0), (d, g, 1184, "SQ_WAIT_INST_LDS", 20.0),
                 (d, g, 1184, "TA_FLAT_READ_WAVEFRONTS_sum", 77.0)]
    write_run(tmp_path, rows)
    md = PR.lds_ta_markdown(str(tmp_path), "t")
    assert "| gemm_bf16w<true, true> | 1184 | 2 | 0.250 | 0.020 | 0.50 | 77 |" in md


def test_committed_summaries_are_whole():
    """Every committed summary opens with its title and the command that made it; the traffic
    summaries still carry the figure and the source digest the bench reads."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    names = sorted(n for n in os.listdir(root) if n.endswith(".md"))
    assert names
    for n in names:
        with open(os.path.join(root, n)) as f:
            text = f.read()
        assert text.startswith("# "), n
        assert "```\ncd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT\nrocprofv3 " in text, n
        if n.endswith("_traffic.md"):
            t, d = PR.stored_traffic(os.path.join(root, n))
            assert t > 0 and len(d) == 16, n
