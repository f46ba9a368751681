"""Host logic of bench.py's profiler helpers: labelling rocprofv3 dispatches
with the launch of the timed step they belong to (no GPU needed)."""
import bench


def rows_for(steps, layers, gemm_in_kernels):
    rows, d = [], 0
    names = []
    for _ in range(steps):
        names += ["void w8a16::gemv_kernel<4>(...)"] * (2 * layers)
        names += gemm_in_kernels
        names += ["void w8a16::(anonymous namespace)::gemm_kernel<128>(...)"]
        names += ["void at::native::elementwise_kernel(...)"]
    for n in names:
        d += 1
        rows.append({"Dispatch_Id": str(d), "Kernel_Name": n})
    return rows


def test_labels_follow_dispatch_order():
    wide = "void w8a16::wide_gemm_kernel<true>(...)"
    tile = "void w8a16::(anonymous namespace)::gemm_kernel<128>(...)"
    comb = "void w8a16::(anonymous namespace)::combine_kernel(...)"
    rows = rows_for(2, 3, [wide, tile, comb])
    labels = bench.label_dispatches(rows, layers=3)
    per_step = ["gemv_in_proj"] * 3 + ["gemv_out_proj"] * 3 + [
        "gemm_in_proj:wide_gemm_kernel<true>", "gemm_in_proj:gemm_kernel<128>", "gemm_in_proj:combine_kernel",
        "gemm_out_proj:gemm_kernel<128>", None]
    assert labels == per_step * 2


def test_labels_ignore_row_order_and_repeats():
    # counter CSVs hold one row per dispatch and counter, in any order
    rows = rows_for(1, 2, ["void w8a16::wide_gemm_kernel<true>(...)"])
    doubled = list(reversed(rows)) + rows
    labels = bench.label_dispatches(doubled, layers=2)
    by_id = {}
    for r, lab in zip(doubled, labels):
        by_id.setdefault(r["Dispatch_Id"], set()).add(lab)
    assert all(len(v) == 1 for v in by_id.values())
    assert by_id["5"] == {"gemm_in_proj:wide_gemm_kernel<true>"}
    assert by_id["6"] == {"gemm_out_proj:gemm_kernel<128>"}


def test_binding_roof_is_the_larger_time():
    assert abs(bench.binding_roof_s(8e12, 0) - 1.0) < 1e-12          # 8 TB at 8 TB/s
    assert abs(bench.binding_roof_s(0, 2516.6e12) - 1.0) < 1e-12     # 2516.6 Tflop at the MFMA peak
    assert abs(bench.binding_roof_s(8e12, 2 * 2516.6e12) - 2.0) < 1e-12


def test_summarize_sq_on_synthetic_csvs(tmp_path, capsys):
    import csv
    layers = 2
    gemv = "void w8a16::gemv_kernel<4>(...)"
    wide = "void w8a16::wide_gemm_kernel<0, false>(...)"
    tile = "void w8a16::gemm_kernel_128(...)"
    names = [gemv] * 4 + [wide, tile, tile]
    pmc, trace = tmp_path / "p_counter_collection.csv", tmp_path / "t_kernel_trace.csv"
    with open(pmc, "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, n in enumerate(names, 1):
            for c, v in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6), ("GRBM_GUI_ACTIVE", 8e5),
                         ("SQ_VALU_MFMA_BUSY_CYCLES", 2.048e8)):
                for _ in range(2):                   # two rows per counter: summed
                    w.writerow({"Dispatch_Id": d, "Kernel_Name": n, "Counter_Name": c, "Counter_Value": v / 2})
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d, n in enumerate(names, 1):
            w.writerow({"Dispatch_Id": d, "Kernel_Name": n, "Start_Timestamp": 0, "End_Timestamp": 100000})
    bench.summarize_sq([str(pmc), str(trace)], layers=layers)
    out = capsys.readouterr().out
    # GUI 8e5 over 8 XCDs in 100 us: 1 GHz; busy 2.048e8 over 1e5 cycles x 1024 SIMDs: 2.0
    assert "| gemm_in_proj:wide_gemm_kernel<0, false> | 1 | 100.0 |" in out
    assert "| 1.00 | 2.000 | 0.833 |" in out
    assert "gemm_in_proj: MOPS_BF16 x 512 = 1.024e+09" in out
