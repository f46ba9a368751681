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
