"""The measurement code of bench.py on synthetic rocprofv3 CSV files (CPU only): the kernel-kind
classification of a trace, the kernel-time summary (launches that overlapped another kernel
or covered part of the batch left out, each stream classified on its own), the counter summary (MFMA busy over
GRBM_GUI_ACTIVE summed across the 8 XCDs) and the calibrated HBM traffic."""
import csv
import re

import pytest

import bench

QKV = "void mb::gemm_kernel<__bf16, 256, 256, 2, 4, 1, 1, 2, 128>(mb::GemmArgs)"
QKV_MANGLED = "_ZN2mb11gemm_kernelIDF16bLi256ELi256ELi2ELi4ELi1ELi1ELi2ELi128EEEvNS_8GemmArgsE"
RESID = "void mb::gemm_kernel<__bf16, 128, 128, 2, 2, 2, 2, 2, 128>(mb::GemmArgs)"
GEGLU = "void mb::gemm_kernel<__bf16, 256, 256, 2, 4, 3, 1, 2, 128>(mb::GemmArgs)"
ATTN = "void mb::attn_kernel<__bf16, 1>(__bf16 const*, __bf16*, int const*, int, int, int, int, int, float)"
EMBED = "mb::embed_ln_kernel(int const*, int, mb::MetaView)"
FINAL = "mb::final_ln_kernel(float const*)"
OTHER = "mb::pack_meta_kernel(int const*)"


def forward_names(layers=4):
    names = [OTHER, EMBED]
    for _ in range(layers):
        names += [QKV, ATTN, RESID, GEGLU, RESID]
    return names + [FINAL]


def test_kernel_matches_both_name_forms():
    assert bench.kernel_matches("qkv_rope", QKV) and bench.kernel_matches("qkv_rope", QKV_MANGLED)
    assert not bench.kernel_matches("wi_geglu", QKV)
    assert bench.kernel_matches("wi_geglu", GEGLU) and bench.kernel_matches("wo_resid", RESID)
    assert bench.kernel_matches("final_pool", FINAL) and not bench.kernel_matches("final_pool", OTHER)


def test_classify_orders_attention_and_residual_kinds_within_each_forward():
    kinds = bench.classify_dispatches(forward_names() * 2)
    one = [None, "embed_ln"]
    for layer in range(4):
        att = "attn_global" if layer % 3 == 0 else "attn_local"
        one += ["qkv_rope", att, "wo_resid", "wi_geglu", "wo2_resid"]
    one += ["final_pool"]
    assert kinds == one * 2  # the embedding launch restarts the layer count


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


TRACE_HEADER = ["Kind", "Stream_Id", "Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                "End_Timestamp", "Grid_Size_X"]


def test_profile_summary_leaves_out_overlapping_launches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "SUMMARY_DIR", str(tmp_path / "sum"))
    (tmp_path / "sum").mkdir()
    wid = 3  # one 8192-token sequence: the embedding grid identifies its trace
    grid = ((8192 + 7) // 8) * 256
    rows, t, d = [], 1000, 0

    def launch(name, dur, stream=0, start=None, grid_x=1):
        nonlocal t, d
        d += 1
        s0 = t if start is None else start
        rows.append(["KERNEL_DISPATCH", stream, d, name, s0, s0 + dur, grid_x])
        if start is None:
            t = s0 + dur + 10

    # one serial forward: QKV launches of 100 ns each
    for name in forward_names():
        launch(name, 100, grid_x=grid if name == EMBED else 64)
    # a launch on part of the batch (smaller grid, as a grouped forward's): left out
    launch(QKV, 40, grid_x=16)
    # a forward on fewer sequences (a smaller embedding grid, as the batch-size sweep's) whose
    # kernels have the whole batch's grids (a persistent GEMM's one workgroup per CU): left out
    for name in forward_names():
        launch(name, 50, grid_x=grid // 2 if name == EMBED else 64)
    # a second stream's forward overlapping a first-stream one (QKV 1000 ns, both left out)
    base = t
    for k, name in enumerate(forward_names()):
        launch(name, 1000, stream=1, start=base + 20 * k, grid_x=grid if name == EMBED else 1)
        launch(name, 1000, stream=2, start=base + 20 * k + 5, grid_x=grid if name == EMBED else 1)
    tdir = tmp_path / "trace"
    tdir.mkdir()
    _write(tdir / "7_kernel_trace.csv", TRACE_HEADER, rows)
    bench.profile_summary(str(tdir), wid, ["cmd"])
    md = (tmp_path / "sum" / "kernel_stats_L8192_bf16.md").read_text()
    line = next(ln for ln in md.splitlines() if ln.startswith("| qkv_rope |"))
    cells = [c.strip() for c in line.split("|")]
    assert cells[2] == "4" and float(cells[3]) == pytest.approx(0.1)  # 4 launches of 100 ns
    m = re.search(r"\((\d+) launches\)|legs: (\d+) launches", md)
    assert m and int(m.group(2)) == 2 * len(forward_names())
    # the grid-16 launch and the 22 classified launches of the smaller forward
    assert "per-group launches: 23)" in md
    # the attention kinds of the serial forward: layers 0 and 3 global, 1 and 2 local
    g = next(ln for ln in md.splitlines() if ln.startswith("| attn_global |"))
    assert [c.strip() for c in g.split("|")][2] == "2"


def test_counter_summary_scales_grbm_by_the_xcd_count(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "SUMMARY_DIR", str(tmp_path))
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    # 2 dispatches of the QKV GEMM: 1000 GPU-busy cycles per XCD (8000 summed), MFMA busy
    # cycles = 0.25 of 1000 cycles x 1024 SIMDs, exactly the algorithmic MFMA count of the
    # 28,186-token workload (32,768 flops each), 3.5 other VALU instructions per MFMA
    n_mfma = 2.0 * 28186 * 768 * 2304 / 32768
    for disp in (1, 2):
        rows += [[disp, QKV, "GRBM_GUI_ACTIVE", 8000.0],
                 [disp, QKV, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1000 * 1024],
                 [disp, QKV, "SQ_INSTS_MFMA", n_mfma], [disp, QKV, "SQ_INSTS_VALU", 4.5 * n_mfma]]
    d = tmp_path / "pmc"
    d.mkdir()
    _write(d / "r_counter_collection.csv", header, rows)
    bench.counter_summary([str(d)], 4, ["cmd"])
    md = (tmp_path / "counters_s64_loguniform32-2048_bf16.md").read_text()
    line = next(ln for ln in md.splitlines() if ln.startswith("| qkv_rope |"))
    cells = [c.strip() for c in line.split("|")]
    assert cells[2] == "2" and cells[3] == "0.250" and cells[4] == "3.50" and cells[5] == "1.000"


def test_traffic_summary_calibrates_on_the_streaming_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "SUMMARY_DIR", str(tmp_path))
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    calib = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    kib = bench.CALIB_BYTES / 1024.0
    for counter, calib_read, kernel_read in (("FETCH_SIZE", kib / 2, 1000.0),
                                             ("WRITE_SIZE", kib, 300.0)):
        d = tmp_path / counter
        d.mkdir()
        # two forwards' worth of the kinds around the QKV dispatches, which alone are counted
        rows = [[1, EMBED, counter, 5.0], [2, QKV, counter, kernel_read],
                [3, ATTN, counter, 7.0], [4, calib, counter, calib_read],
                [5, EMBED, counter, 5.0], [6, QKV, counter, kernel_read]]
        _write(d / "r_counter_collection.csv", header, rows)
    bench.traffic_summary(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"), "qkv_rope",
                          "w", ["cmd"])
    import json
    out = json.loads((tmp_path / "traffic_qkv_rope_w.json").read_text())
    # the fetch counter reads half the calibration bytes: scale 2; the write counter all: 1
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    assert out["hbm_bytes_per_launch"] == pytest.approx((2 * 1000.0 + 300.0) * 1024)
    # global attention shares its symbol with local attention: classified by its order
    bench.traffic_summary(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"), "attn_global",
                          "w", ["cmd"])
    out = json.loads((tmp_path / "traffic_attn_global_w.json").read_text())
    assert out["dispatches"] == [1, 1]
    assert out["hbm_bytes_per_launch"] == pytest.approx((2 * 7.0 + 7.0) * 1024)
