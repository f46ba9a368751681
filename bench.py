"""Benchmark of the w8a16 block-scaled FP8 projections on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  * decode: one token through LAYERS layers of the Mamba-2 projections, i.e.
    LAYERS in_proj GEMVs (M=1, K=4096, N=18560) and LAYERS out_proj GEMVs
    (M=1, K=8192, N=4096), each layer with its own weight copy, and
  * prefill: one 1024-token prompt through in_proj and out_proj with the
    prefill GEMM (M=1024),
on seeded random inputs (A ~ N(0,1) BF16; weights N(0, 0.02) quantized per
128x128 block to E4M3 with BF16 scales). Inputs are resident in HBM before
timing starts. The weight copies (layers) rotate over more than 1 GB, so
every GEMV reads its weights from HBM rather than from the 256 MB Infinity
Cache, as decode over a real layer stack does.

The JSON line reports the decode GEMV's HBM bandwidth as `value` (GB/s over
both projections: algorithmic bytes / kernel time) and the prefill GEMM's
TFLOP/s under `prefill`, each with a roofline object for the pair of
launches it is quoted on (in_proj + out_proj), and `launches` has one
roofline object per launch of the step. Kernel times come from HIP events
on the launch stream: the GEMVs of one projection run back to back between
two events (so the average launch duration is not inflated by per-event
overhead), the GEMMs each between their own two events. `cpu_baseline` times
the CPU oracle on a bounded sample of the same workloads. `large_layer`
(outside the timed step) times the 8192-token prefill GEMMs and the M = 1
GEMVs of the hidden-8192 layer (in_proj K=8192 N=35072, out_proj K=16384
N=8192). `few_tokens` (outside the timed step) reports the same projections
at M = 2..16 through the GEMV entry point (the multi-sequence decode
workloads) and at M = 32..256 through the GEMM, without and with a
workspace (w8a16_gemm_ws), each against its binding roof max(bytes / HBM
peak, flop / MFMA peak).
`read_floor` (outside the timed step) times a plain read of each projection's
weight bytes (w8a16_hbm_read, several launch shapes, the same rotating copies
and event timing as the GEMVs): the floor the GEMV pair is compared against.
`vendor_bf16_gemm` (outside the timed step, context only) times torch.matmul
(hipBLASLt) in bf16 on the same prefill shapes with the weights dequantized.
`layer_ends` (outside the timed step) times the norm prologues and the
residual epilogue: fused into the decode GEMV against the unfused chain, and
the prefill norms and residual GEMM at M = 1024. `decode_layer` times one
Mamba-2 layer's whole decode step for one token (fused in_proj, conv1d
update, SSM decode, fused out_proj) and the conv / SSM kernels alone.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-few-tokens]
                    [--no-layer-ends] [--no-large-layer] [--no-read-floor] [--no-vendor]

Profile helpers (read rocprofv3 CSV output; no GPU needed):
    python bench.py --summarize-trace <dir>/<name>_kernel_trace.csv
    python bench.py --summarize-counters <fetch counter_collection.csv> <write counter_collection.csv>
The second writes profiles/hbm_traffic.json, which `roofline.traffic` reads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from gemm_mamba_ssm_amd import binding, inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
ROTATE_BYTES = 1.2e9            # weight copies per projection span at least this much
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "gemv": ["gemm_mamba_ssm_amd/csrc/w8a16_gemv.hip", "gemm_mamba_ssm_amd/csrc/w8a16_device.h"],
    "gemm": ["gemm_mamba_ssm_amd/csrc/w8a16_gemm.hip", "gemm_mamba_ssm_amd/csrc/w8a16_gemm_wide.hip",
             "gemm_mamba_ssm_amd/csrc/w8a16_device.h"],
}
METRIC = "M=1 GEMV HBM GB/s (%peak) + 1k-token prefill GEMM TFLOP/s (%MFMA peak)"
CALIBRATION_BYTES = 256 << 20   # the plain copy run with --copy-calibration reads and writes this much

# Launches of the timed step, told apart in profiler output by kernel name and
# dispatch order: every step issues LAYERS in_proj GEMVs, LAYERS out_proj GEMVs,
# then the in_proj GEMM and the out_proj GEMM, and nothing else in the process
# launches these kernels. The 1024-token in_proj GEMM is two kernels (256 x 256
# tiles over the first 16384 columns, then the k-split 128 x 128 tiles over the
# rest), the out_proj GEMM one: of the GEMM dispatches that follow a step's
# GEMVs, the last is the out_proj's and the others the in_proj's.
LAUNCHES = ["gemv_in_proj", "gemv_out_proj", "gemm_in_proj", "gemm_out_proj"]
DEFAULT_LAYERS = 8
NORM_GROUP = 1024               # the gated norm in groups: Mamba-2 with d_inner 8192 and 8 groups


def _kernel_kind(name):
    if "gemv" in name and "kernel" in name:
        return "gemv"
    if "gemm_kernel" in name or "combine_kernel" in name or "skinny" in name:
        return "gemm"
    return None


def label_dispatches(rows, layers=DEFAULT_LAYERS):
    """Label each rocprofv3 CSV row (one per dispatch, or per dispatch and
    counter) with its launch, from the dispatch order; None for other kernels.
    GEMM labels carry the kernel too: 'gemm_in_proj:<kernel>'."""
    names = {int(r["Dispatch_Id"]): r["Kernel_Name"] for r in rows}
    order = sorted(names)
    labels_by_id = {}
    gemv_seen = 0
    pending = []                                 # GEMM dispatches since the last GEMV

    def flush():
        for j, d in enumerate(pending):
            proj = "gemm_out_proj" if j == len(pending) - 1 else "gemm_in_proj"
            labels_by_id[d] = f"{proj}:{short_name(names[d])}"
        pending.clear()

    for d in order:
        kind = _kernel_kind(names[d])
        if kind == "gemv":
            flush()
            labels_by_id[d] = "gemv_in_proj" if (gemv_seen // layers) % 2 == 0 else "gemv_out_proj"
            gemv_seen += 1
        elif kind == "gemm":
            pending.append(d)
        else:
            labels_by_id[d] = None
    flush()
    return [labels_by_id[int(r["Dispatch_Id"])] for r in rows]


LARGE_REPS, LARGE_L = 5, 4                     # large_layer_report's repetitions and GEMVs per repetition


def label_large(rows, reps=LARGE_REPS, L=LARGE_L):
    """Labels for a --large-layer-only run, which issues per projection (in_proj,
    then out_proj) 1 + reps GEMMs and then L + reps * L GEMVs."""
    names = {int(r["Dispatch_Id"]): r["Kernel_Name"] for r in rows}
    labels_by_id, gemvs, gemms = {}, 0, 0
    per_proj_gemv = L + reps * L
    for d in sorted(names):
        kind = _kernel_kind(names[d])
        if kind == "gemm":
            proj = "in_proj" if gemms < 1 + reps else "out_proj"
            labels_by_id[d] = f"gemm8k_{proj}:{short_name(names[d])}"
            gemms += 1
        elif kind == "gemv":
            labels_by_id[d] = "gemv_large_" + ("in_proj" if gemvs < per_proj_gemv else "out_proj")
            gemvs += 1
        else:
            labels_by_id[d] = None
    return [labels_by_id[int(r["Dispatch_Id"])] for r in rows]


def summarize_sq(csvs, layers=DEFAULT_LAYERS, large=False):
    """Matrix-core and LDS counters per GEMM launch (and per kernel of it) from
    rocprofv3 --pmc runs (several CSVs, one per pass). Per dispatch, counters
    are summed over the GPU; GRBM_GUI_ACTIVE over its 8 XCDs."""
    XCDS, SIMDS = 8, 4
    per = {}                                     # (label) -> counter -> [values per dispatch]
    dur = {}
    for path in csvs:
        rows = _read_csv(path)
        labels = label_large(rows) if large else label_dispatches(rows, layers)
        if rows and "Counter_Name" not in rows[0]:           # a kernel trace of one of the runs
            for r, lab in zip(rows, labels):
                if lab is not None and lab.startswith("gemm"):
                    dur.setdefault(lab, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
            continue
        acc = {}
        for r, lab in zip(rows, labels):
            if lab is None or not lab.startswith("gemm"):
                continue
            key = (lab, int(r["Dispatch_Id"]), r["Counter_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        for (lab, _, c), v in acc.items():
            per.setdefault(lab, {}).setdefault(c, []).append(v)
    flops = {}
    wl = inputs.WORKLOADS["prefill_8k_large" if large else "prefill_1k"]
    for p in wl:
        flops[("gemm8k_" if large else "gemm_") + p.name] = p.flops()
    cus = 256
    print("| launch : kernel | dispatches | median us | MOPS_BF16 x 512 / (2MNK) | clock GHz (GUI/XCD per us) | "
          "MFMA busy (of GUI cycles) | MFMA busy cycles / (us x 2.4 GHz) | LDS bank conflict / LDS active | "
          "LDS cmd FIFO full / LDS active |")
    print("|---|---|---|---|---|---|---|---|---|")
    launch_mops = {}
    for lab in sorted(per):
        c = {k: float(np.median(v)) for k, v in per[lab].items()}
        n = max(len(v) for v in per[lab].values())
        base = lab.split(":")[0]
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        if mops is not None:
            launch_mops[base] = launch_mops.get(base, 0.0) + mops
        gui = c.get("GRBM_GUI_ACTIVE")
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        util = busy / (gui / XCDS * cus * SIMDS) if gui and busy is not None else None
        lds = c.get("SQ_LDS_IDX_ACTIVE")
        conf = c.get("SQ_LDS_BANK_CONFLICT")
        fifo = c.get("SQ_LDS_CMD_FIFO_FULL")
        t = float(np.median(dur[lab])) if lab in dur else None

        def f(x, fmt):
            return format(x, fmt) if x is not None else "-"
        print(f"| {lab} | {n} | {f(t, '.1f')} | {f(mops * 512 / flops[base] if mops is not None and base in flops else None, '.4f')} | "
              f"{f(gui / XCDS / t / 1e3 if gui and t else None, '.2f')} | {f(util, '.3f')} | "
              f"{f(busy / (t * 1e-6 * 2.4e9 * cus * SIMDS) if busy is not None and t else None, '.3f')} | "
              f"{f(conf / lds if lds and conf is not None else None, '.4f')} | {f(fifo / lds if lds and fifo is not None else None, '.4f')} |")
    for base, m in sorted(launch_mops.items()):
        if base in flops:
            print(f"\n{base}: MOPS_BF16 x 512 = {m * 512:.6g} flop per launch, 2MNK = {flops[base]:.6g} "
                  f"(ratio {m * 512 / flops[base]:.4f})")


def short_name(name):
    return name.replace("(anonymous namespace)::", "").replace("void ", "").replace("w8a16::", "").split("(")[0]


def source_digest(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str, launch: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when missing or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("kernels", {}).get(launch)
    if not entry or entry.get("source_digest") != source_digest(kind):
        return None
    return entry.get("hbm_bytes_per_launch")


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_trace(path, layers=DEFAULT_LAYERS, large=False):
    """Average duration per launch (and per other kernel) from a rocprofv3 kernel_trace.csv."""
    rows = _read_csv(path)
    by = {}
    for r, lab in zip(rows, label_large(rows) if large else label_dispatches(rows, layers)):
        name = r["Kernel_Name"]
        grid = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1) * int(r.get("Grid_Size_Z", 1) or 1)
        by.setdefault((lab or "", name, grid), []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("| launch | kernel | grid (threads) | dispatches | mean us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (lab, name, grid), d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        short = short_name(name)
        print(f"| {lab} | {short} | {grid} | {len(d)} | {np.mean(d) / 1e3:.2f} | "
              f"{np.min(d) / 1e3:.2f} | {np.max(d) / 1e3:.2f} |")


def summarize_counters(fetch_csv, write_csv, layers=DEFAULT_LAYERS):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for a plain copy of known size."""

    def per_launch(path, counter):
        vals, calib = {}, []
        rows = [r for r in _read_csv(path) if r["Counter_Name"] == counter]
        for r, lab in zip(rows, label_dispatches(rows, layers)):
            name, grid, v = r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])
            if "neg" in name and grid >= CALIBRATION_BYTES // 4 // 8:
                calib.append(v)
            if lab is not None:
                vals.setdefault(lab, []).append(v)
        if not calib:
            raise SystemExit(f"no calibration copy found in {path}")
        factor = (CALIBRATION_BYTES / 1024) / float(np.median(calib))
        per = {k: float(np.median(v)) for k, v in vals.items()}
        launch = {}                              # a launch's kernels add up
        for k, v in per.items():
            launch[k.split(":")[0]] = launch.get(k.split(":")[0], 0.0) + v
        return launch, factor

    fetch, f_fac = per_launch(fetch_csv, "FETCH_SIZE")
    write, w_fac = per_launch(write_csv, "WRITE_SIZE")
    rec = {"source": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, of "
                     "`python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-few-tokens --no-layer-ends --no-large-layer "
                     "--copy-calibration`",
           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4), "kernels": {}}
    for lab in fetch:
        kind = lab.split("_")[0]
        kib_f, kib_w = fetch[lab], write.get(lab, 0.0)
        rec["kernels"][lab] = {
            "fetch_kib": kib_f, "write_kib": kib_w,
            "hbm_bytes_per_launch": int(round((kib_f * f_fac + kib_w * w_fac) * 1024)),
            "source_digest": source_digest(kind)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec, indent=1, sort_keys=True))


def to_dev(a: np.ndarray, dtype, device):
    raw = np.ascontiguousarray(a)
    view = raw.view(np.int16) if raw.dtype == np.uint16 else raw
    return torch.from_numpy(view.copy()).view(dtype).to(device)


class Projection:
    """Device buffers of one projection: rotating weight copies, decode and prefill operands."""

    def __init__(self, p_dec, p_pre, device):
        assert (p_dec.N, p_dec.K, p_dec.seed_w) == (p_pre.N, p_pre.K, p_pre.seed_w)
        self.p_dec, self.p_pre = p_dec, p_pre
        A1, W, S = inputs.make(p_dec)
        Ap, _, _ = inputs.make(p_pre)
        wq = to_dev(W, torch.uint8, device)
        sc = to_dev(S, torch.bfloat16, device)
        self.copies = max(2, math.ceil(ROTATE_BYTES / W.nbytes))   # distinct layers' weights
        self.W = [wq] + [wq.clone() for _ in range(self.copies - 1)]
        self.S = [sc] + [sc.clone() for _ in range(self.copies - 1)]
        self.A1 = to_dev(A1, torch.bfloat16, device)
        self.Ap = to_dev(Ap, torch.bfloat16, device)
        self.out1 = torch.empty((p_dec.M, p_dec.N), dtype=torch.bfloat16, device=device)
        self.outp = torch.empty((p_pre.M, p_pre.N), dtype=torch.bfloat16, device=device)

    def gemv(self, i, stream):
        return binding.gemv_raw(self.A1.data_ptr(), self.W[i % self.copies].data_ptr(),
                                self.S[i % self.copies].data_ptr(), self.out1.data_ptr(),
                                self.p_dec.M, self.p_dec.N, self.p_dec.K, stream)

    def gemm(self, i, stream):
        return binding.gemm_raw(self.Ap.data_ptr(), self.W[i % self.copies].data_ptr(),
                                self.S[i % self.copies].data_ptr(), self.outp.data_ptr(),
                                self.p_pre.M, self.p_pre.N, self.p_pre.K, stream)


# Launch shapes (threads, loads per lane) of the plain-read floor: the fastest
# one-shot shapes for the two weight sizes on MI355X, and the GEMVs' own.
READ_SHAPES = ((512, 2), (256, 8), (64, 8), (256, 2), (128, 8), (256, 4), (512, 4), (512, 8))


def read_floor_report(projs, device, stream, L, check, gemv_us, reps=10):
    """Outside the timed step: the plain read of each projection's weight
    bytes (w8a16_hbm_read over the same rotating weight copies the GEMVs
    read, L back-to-back launches between two events, like the GEMVs), at the
    launch shapes in READ_SHAPES; the fastest is the floor the GEMV is
    compared against."""
    sh = stream.cuda_stream
    sink = torch.zeros(1024, dtype=torch.int32, device=device)
    out = {"unit": "us per launch (HIP events over L back-to-back launches, weight copies rotated)"}
    best = []
    for proj, g_us in zip(projs, gemv_us):
        nbytes = proj.p_dec.N * proj.p_dec.K
        rows = {}
        for threads, loads in READ_SHAPES:
            def launch(i):
                check(binding.hbm_read_raw(proj.W[i % proj.copies].data_ptr(), nbytes, threads, loads,
                                           sink.data_ptr(), sh), "hbm_read")
            for i in range(L):
                launch(i)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
            for r in range(reps):
                ev[2 * r].record(stream)
                for i in range(L):
                    launch(r * L + i)
                ev[2 * r + 1].record(stream)
            torch.cuda.synchronize()
            t = float(np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e-3 for r in range(reps)])) / L
            rows[f"{threads}x{loads}"] = round(t * 1e6, 3)
        shape, t_best = min(rows.items(), key=lambda kv: kv[1])
        best.append(t_best)
        out[proj.p_dec.name] = {"weight_bytes": nbytes, "us_by_shape (threads x loads per lane)": rows,
                                "best_us": t_best, "best_shape": shape,
                                "frac_of_hbm_peak": round(nbytes / (t_best * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "gemv_us": round(g_us, 3), "gemv_over_floor": round(g_us / t_best, 3)}
    assert not bool(sink.any()), "the read helper wrote to its sink"
    b = sum(p.p_dec.N * p.p_dec.K for p in projs)
    out["pair"] = {"floor_us": round(sum(best), 3),
                   "floor_frac_of_hbm_peak": round(b / (sum(best) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "gemv_us": round(sum(gemv_us), 3), "gemv_over_floor": round(sum(gemv_us) / sum(best), 3)}
    return out


FEW_TOKEN_GEMV_M = (2, 4, 8, 16)            # multi-sequence decode (w8a16_gemv)
FEW_TOKEN_GEMM_M = (32, 64, 128, 256)        # skinny prefill / verify (w8a16_gemm)


def binding_roof_s(nbytes, flop):
    """Time at the binding roof: the larger of bytes at the HBM peak and flop
    at the dense bf16 MFMA peak (seconds)."""
    return max(nbytes / (HBM_PEAK_GBS * 1e9), flop / (BF16_PEAK_TFLOPS * 1e12))


def few_token_report(projs, device, stream, L, check, reps=10):
    """Outside the timed step: the same projections at a few tokens, through
    w8a16_gemv (M = 2..16, the multi-sequence decode workloads) and w8a16_gemm
    (M = 32..256), the GEMM also through w8a16_gemm_ws with a workspace (the
    k-split schedule of shapes whose tiles do not fill the GPU). Weight copies
    rotate as in the decode step; each figure is the mean over `reps` runs of
    L back-to-back launches between two events. `roof` is the fraction of the
    binding roof max(bytes / 8 TB/s, flop / 2.5166 PFLOP/s)."""
    sh = stream.cuda_stream
    out = {"unit": "us per launch; GB/s = algorithmic bytes / time; roof = binding-roof time / time, "
                   "binding roof = max(bytes / 8 TB/s, flop / 2516.6 TFLOP/s)",
           "gemv": [], "gemm": [], "gemm_ws": []}
    for entry, ms in (("gemv", FEW_TOKEN_GEMV_M), ("gemm", FEW_TOKEN_GEMM_M), ("gemm_ws", FEW_TOKEN_GEMM_M)):
        for m in ms:
            row = {"M": m}
            for proj in projs:
                p = proj.p_dec
                if entry == "gemv":
                    (q,) = [x for x in inputs.WORKLOADS[f"multiseq_m{m}"] if x.name == p.name]
                    A = inputs.make(q)[0]
                else:
                    A = inputs.activations(m, p.K, 5000 + m)
                dA = to_dev(A, torch.bfloat16, device)
                dO = torch.empty((m, p.N), dtype=torch.bfloat16, device=device)
                ws = binding.gemm_workspace(m, p.N, p.K, device) if entry == "gemm_ws" else None

                def launch(i):
                    w, s_ = proj.W[i % proj.copies].data_ptr(), proj.S[i % proj.copies].data_ptr()
                    if entry == "gemv":
                        st = binding.gemv_raw(dA.data_ptr(), w, s_, dO.data_ptr(), m, p.N, p.K, sh)
                    elif entry == "gemm":
                        st = binding.gemm_raw(dA.data_ptr(), w, s_, dO.data_ptr(), m, p.N, p.K, sh)
                    else:
                        st = binding.gemm_ws_raw(dA.data_ptr(), w, s_, dO.data_ptr(), m, p.N, p.K,
                                                 ws.data_ptr() if ws is not None else 0,
                                                 ws.numel() if ws is not None else 0, sh)
                    check(st, entry)

                for i in range(L):
                    launch(i)
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
                for r in range(reps):
                    ev[2 * r].record(stream)
                    for i in range(L):
                        launch(r * L + i)
                    ev[2 * r + 1].record(stream)
                torch.cuda.synchronize()
                t = np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e-3 for r in range(reps)]) / L
                nbytes = p.N * p.K + 2 * (-(-p.N // 128)) * (-(-p.K // 128)) + 2 * m * p.K + 2 * m * p.N
                flop = 2 * m * p.N * p.K
                row[p.name] = {"us": round(t * 1e6, 2), "GB/s": round(nbytes / t / 1e9, 1),
                               "TFLOP/s": round(flop / t / 1e12, 2),
                               "roof": round(binding_roof_s(nbytes, flop) / t, 4),
                               "workspace_bytes": ws.numel() if ws is not None else 0}
                if entry != "gemm_ws":
                    del row[p.name]["workspace_bytes"]
            out[entry].append(row)
    return out


def large_layer_report(device, stream, check, reps=LARGE_REPS, L=LARGE_L):
    """Outside the timed step: the hidden-8192 layer (in_proj K=8192 N=35072,
    out_proj K=16384 N=8192): the 8192-token prefill GEMM of each projection
    (mean over `reps` launches, each between two events) and the M = 1 decode
    GEMV (L back-to-back launches over rotating weight copies, `reps` times),
    on the same seeded generator as the tests."""
    sh = stream.cuda_stream
    out = {"unit": "us per launch", "workload": "prefill_8k_large (M=8192) and decode_m1_large (M=1)"}
    for p_pre, p_dec in zip(inputs.WORKLOADS["prefill_8k_large"], inputs.WORKLOADS["decode_m1_large"]):
        A, W, S = inputs.make(p_pre)
        dA, dW, dS = to_dev(A, torch.bfloat16, device), to_dev(W, torch.uint8, device), to_dev(S, torch.bfloat16, device)
        del A
        dO = torch.empty((p_pre.M, p_pre.N), dtype=torch.bfloat16, device=device)

        def gemm():
            check(binding.gemm_raw(dA.data_ptr(), dW.data_ptr(), dS.data_ptr(), dO.data_ptr(), p_pre.M, p_pre.N,
                                   p_pre.K, sh), "gemm")

        gemm()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            ev[2 * r].record(stream)
            gemm()
            ev[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        t = float(np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e-3 for r in range(reps)]))
        f = p_pre.flops()
        rec = {"gemm": {"M": p_pre.M, "us": round(t * 1e6, 1), "TFLOP/s": round(f / t / 1e12, 1),
                        "frac_of_mfma_peak": round(f / t / 1e12 / BF16_PEAK_TFLOPS, 4)}}
        del dA, dO
        copies = max(2, math.ceil(ROTATE_BYTES / W.nbytes))
        Ws = [dW] + [dW.clone() for _ in range(copies - 1)]
        a1 = to_dev(inputs.make(p_dec)[0], torch.bfloat16, device)
        o1 = torch.empty((1, p_dec.N), dtype=torch.bfloat16, device=device)

        def gemv(i):
            check(binding.gemv_raw(a1.data_ptr(), Ws[i % copies].data_ptr(), dS.data_ptr(), o1.data_ptr(), 1,
                                   p_dec.N, p_dec.K, sh), "gemv")

        for i in range(L):
            gemv(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            ev[2 * r].record(stream)
            for i in range(L):
                gemv(r * L + i)
            ev[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        t = float(np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e-3 for r in range(reps)])) / L
        b = p_dec.bytes_moved()
        rec["gemv"] = {"M": 1, "us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                       "frac_of_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4), "weight_copies_rotated": copies}
        out[p_pre.name] = rec
        del Ws, dW
        torch.cuda.empty_cache()
    return out


def vendor_gemm_report(device, stream, reps=5):
    """Context, outside the timed step: the vendor library's plain bf16 x bf16
    GEMM (torch.matmul, which calls hipBLASLt) on the prefill shapes, with the
    same activations and the dequantized weights rounded to BF16 ([K, N]
    contiguous). Not this library's path: it reads twice the weight bytes and
    applies no scales in the kernel; it shows what the chip's own GEMM reaches
    on these shapes at the clock they run at."""
    out = {"unit": "us per launch (HIP events around each launch); frac of 2516.6 TFLOP/s",
           "what": "torch.matmul(A bf16 [M,K], B bf16 [K,N]) with B = bf16(dequantized W)^T"}
    for wl in ("prefill_1k", "prefill_8k_large"):
        for p in inputs.WORKLOADS[wl]:
            A, W, S = inputs.make(p)
            dA = to_dev(A, torch.bfloat16, device)
            del A
            deq = binding.w8a16_dequant(to_dev(W, torch.uint8, device), to_dev(S, torch.bfloat16, device))
            B = deq.to(torch.bfloat16).t().contiguous()
            del deq
            for _ in range(2):
                C = torch.matmul(dA, B)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
            for r in range(reps):
                ev[2 * r].record(stream)
                C = torch.matmul(dA, B)
                ev[2 * r + 1].record(stream)
            torch.cuda.synchronize()
            t = float(np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e-3 for r in range(reps)]))
            f = p.flops()
            out[f"{wl}/{p.name}"] = {"M": p.M, "N": p.N, "K": p.K, "us": round(t * 1e6, 1),
                                     "TFLOP/s": round(f / t / 1e12, 1),
                                     "frac": round(f / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
            del dA, B, C
            torch.cuda.empty_cache()
    return out


def layer_ends_report(projs, device, stream, L, check, reps=10):
    """Outside the timed step: the layer's norm prologues and residual epilogue
    around the projections (forward steps 1, 6 and 8 of the Mamba-2 layer).

    Decode (M = 1): in_proj with its RMSNorm fused (w8a16_gemv_fused) against
    w8a16_rmsnorm + w8a16_gemv; out_proj with the gated norm and the residual
    fused against w8a16_rmsnorm + w8a16_gemv + a torch BF16 add (the unfused
    chain). Prefill (M = 1024): the standalone norms (HBM-bound: x, z read
    once, the activations written once) and the out_proj GEMM with and
    without the residual epilogue. Weight copies rotate as in the decode step;
    times are means over `reps` runs of L launches (or chains) between two
    events, in us."""
    sh = stream.cuda_stream
    eps = inputs.NORM_EPS
    pin, pout = projs
    K_in, K_out = pin.p_dec.K, pout.p_dec.K
    x1 = to_dev(inputs.activations(1, K_in, 6001), torch.bfloat16, device)
    y1 = to_dev(inputs.activations(1, K_out, 6002), torch.bfloat16, device)
    z1 = to_dev(inputs.activations(1, K_out, 6003), torch.bfloat16, device)
    w_in = to_dev(inputs.norm_weight(K_in, 6004), torch.bfloat16, device)
    w_out = to_dev(inputs.norm_weight(K_out, 6005), torch.bfloat16, device)
    r1 = to_dev(inputs.activations(1, pout.p_dec.N, 6006), torch.bfloat16, device)
    a_in = torch.empty((1, K_in), dtype=torch.bfloat16, device=device)
    a_out = torch.empty((1, K_out), dtype=torch.bfloat16, device=device)
    o_in = torch.empty((1, pin.p_dec.N), dtype=torch.bfloat16, device=device)
    o_out = torch.empty((1, pout.p_dec.N), dtype=torch.bfloat16, device=device)
    o_sum = torch.empty_like(o_out)

    def W(p, i):
        return p.W[i % p.copies].data_ptr(), p.S[i % p.copies].data_ptr()

    def in_fused(i):
        w, s_ = W(pin, i)
        check(binding.gemv_fused_raw(x1.data_ptr(), 0, w_in.data_ptr(), eps, w, s_, 0, o_in.data_ptr(),
                                     1, pin.p_dec.N, K_in, sh), "gemv_fused")

    def in_chain(i):
        w, s_ = W(pin, i)
        check(binding.rmsnorm_raw(x1.data_ptr(), 0, w_in.data_ptr(), eps, a_in.data_ptr(), 1, K_in, sh), "rmsnorm")
        check(binding.gemv_raw(a_in.data_ptr(), w, s_, o_in.data_ptr(), 1, pin.p_dec.N, K_in, sh), "gemv")

    def out_fused(i):
        w, s_ = W(pout, i)
        check(binding.gemv_fused_raw(y1.data_ptr(), z1.data_ptr(), w_out.data_ptr(), eps, w, s_, r1.data_ptr(),
                                     o_out.data_ptr(), 1, pout.p_dec.N, K_out, sh), "gemv_fused")

    def out_fused_grouped(i):
        w, s_ = W(pout, i)
        check(binding.gemv_fused_raw(y1.data_ptr(), z1.data_ptr(), w_out.data_ptr(), eps, w, s_, r1.data_ptr(),
                                     o_out.data_ptr(), 1, pout.p_dec.N, K_out, sh, group=NORM_GROUP), "gemv_fused")

    def out_chain(i):
        w, s_ = W(pout, i)
        check(binding.rmsnorm_raw(y1.data_ptr(), z1.data_ptr(), w_out.data_ptr(), eps, a_out.data_ptr(), 1, K_out,
                                  sh), "rmsnorm")
        check(binding.gemv_raw(a_out.data_ptr(), w, s_, o_out.data_ptr(), 1, pout.p_dec.N, K_out, sh), "gemv")
        torch.add(r1, o_out, out=o_sum)

    def timed(fn):
        for i in range(L):
            fn(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            ev[2 * r].record(stream)
            for i in range(L):
                fn(r * L + i)
            ev[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e3 for r in range(reps)]) / L)

    out = {"unit": "us per launch (or per chain of launches)",
           "decode_in_proj": {"fused_norm_gemv": round(timed(in_fused), 2),
                              "rmsnorm_then_gemv": round(timed(in_chain), 2)},
           "decode_out_proj": {"fused_gated_norm_gemv_residual": round(timed(out_fused), 2),
                               f"fused_gated_norm_{K_out // NORM_GROUP}_groups_gemv_residual":
                                   round(timed(out_fused_grouped), 2),
                               "rmsnorm_then_gemv_then_add": round(timed(out_chain), 2)}}

    # prefill: standalone norms and the residual epilogue at M = 1024
    Mp = pin.p_pre.M
    xp = to_dev(inputs.activations(Mp, K_in, 6011), torch.bfloat16, device)
    yp = to_dev(inputs.activations(Mp, K_out, 6012), torch.bfloat16, device)
    zp = to_dev(inputs.activations(Mp, K_out, 6013), torch.bfloat16, device)
    ap_in = torch.empty_like(xp)
    ap_out = torch.empty_like(yp)
    rp = to_dev(inputs.activations(Mp, pout.p_pre.N, 6014), torch.bfloat16, device)
    op = torch.empty((Mp, pout.p_pre.N), dtype=torch.bfloat16, device=device)

    def norm_in(i):
        check(binding.rmsnorm_raw(xp.data_ptr(), 0, w_in.data_ptr(), eps, ap_in.data_ptr(), Mp, K_in, sh), "rmsnorm")

    def norm_out(i):
        check(binding.rmsnorm_raw(yp.data_ptr(), zp.data_ptr(), w_out.data_ptr(), eps, ap_out.data_ptr(), Mp, K_out,
                                  sh), "rmsnorm")

    def norm_out_grouped(i):
        check(binding.rmsnorm_raw(yp.data_ptr(), zp.data_ptr(), w_out.data_ptr(), eps, ap_out.data_ptr(), Mp, K_out,
                                  sh, group=NORM_GROUP), "rmsnorm")

    def gemm_plain(i):
        w, s_ = W(pout, i)
        check(binding.gemm_raw(ap_out.data_ptr(), w, s_, op.data_ptr(), Mp, pout.p_pre.N, K_out, sh), "gemm")

    def gemm_res(i):
        w, s_ = W(pout, i)
        check(binding.gemm_residual_raw(ap_out.data_ptr(), w, s_, rp.data_ptr(), op.data_ptr(), Mp, pout.p_pre.N,
                                        K_out, sh), "gemm_residual")

    t_ni, t_no = timed(norm_in), timed(norm_out)
    b_ni = 2 * Mp * K_in * 2 + 2 * K_in              # x read, a written, weight
    b_no = 3 * Mp * K_out * 2 + 2 * K_out            # y, z read, a written, weight
    out["prefill_rmsnorm_in"] = {"us": round(t_ni, 2), "GB/s": round(b_ni / t_ni / 1e3, 1),
                                 "frac": round(b_ni / t_ni / 1e3 / HBM_PEAK_GBS, 4)}
    out["prefill_gated_rmsnorm_out"] = {"us": round(t_no, 2), "GB/s": round(b_no / t_no / 1e3, 1),
                                        "frac": round(b_no / t_no / 1e3 / HBM_PEAK_GBS, 4)}
    t_ng = timed(norm_out_grouped)
    out[f"prefill_gated_rmsnorm_out_{K_out // NORM_GROUP}_groups"] = {
        "us": round(t_ng, 2), "GB/s": round(b_no / t_ng / 1e3, 1), "frac": round(b_no / t_ng / 1e3 / HBM_PEAK_GBS, 4)}
    out["prefill_out_proj_gemm"] = {"plain": round(timed(gemm_plain), 2), "with_residual": round(timed(gemm_res), 2)}
    return out


SSM_STATE_ROTATE_BYTES = 512 << 20      # SSM states rotate over this much, as the weights do


def decode_layer_report(projs, device, stream, L, check, reps=10):
    """Outside the timed step: one Mamba-2 layer's decode step for one token
    (hidden 4096), every step in this library's kernels: in_proj with its
    RMSNorm fused, the conv1d update on xBC, the SSM decode, out_proj with the
    gated norm (gate z read in place from the in_proj output) and the residual
    fused. Weights and the per-layer conv / SSM states rotate over several
    copies so they come from HBM. Also the conv and SSM kernels alone, with
    their algorithmic bytes (states read and written once)."""
    sh = stream.cuda_stream
    eps = inputs.NORM_EPS
    dims = inputs.MAMBA2_4K
    H, P, S_, G, DC = dims["heads"], dims["head_dim"], dims["state"], dims["groups"], dims["d_conv"]
    d_inner = H * P
    d_xbc = d_inner + 2 * G * S_
    pin, pout = projs
    N_in, K_in, N_out, K_out = pin.p_dec.N, pin.p_dec.K, pout.p_dec.N, pout.p_dec.K
    assert N_in == d_inner + d_xbc + H and K_out == d_inner
    copies = max(2, SSM_STATE_ROTATE_BYTES // (d_inner * S_ * 4))
    h_states = [torch.from_numpy(inputs.ssm_state(1, H, P, S_, 9000)).to(device)]
    h_states += [h_states[0].clone() for _ in range(copies - 1)]
    c_states = [torch.from_numpy(inputs.conv_state(1, d_xbc, DC, 9001)).to(device) for _ in range(copies)]
    cw, cb = (to_dev(a, torch.bfloat16, device) for a in inputs.conv_params(d_xbc, DC, 9002))
    a_log, d_param, dt_bias = (torch.from_numpy(a).to(device) for a in inputs.ssm_params(H, 9003))
    x = to_dev(inputs.activations(1, K_in, 9004), torch.bfloat16, device)
    w_in = to_dev(inputs.norm_weight(K_in, 9005), torch.bfloat16, device)
    w_out = to_dev(inputs.norm_weight(K_out, 9006), torch.bfloat16, device)
    proj = torch.empty((1, N_in), dtype=torch.bfloat16, device=device)      # [z | xBC | dt]
    xbc = torch.empty((1, d_xbc), dtype=torch.bfloat16, device=device)
    y = torch.empty((1, d_inner), dtype=torch.bfloat16, device=device)
    out = torch.empty((1, N_out), dtype=torch.bfloat16, device=device)
    e = 2                                                                    # bytes per BF16 element

    def W(p, i):
        return p.W[i % p.copies].data_ptr(), p.S[i % p.copies].data_ptr()

    def conv(i, h=sh):
        check(binding.conv1d_update_raw(c_states[i % copies].data_ptr(), proj.data_ptr() + e * d_inner, N_in,
                                        cw.data_ptr(), cb.data_ptr(), xbc.data_ptr(), d_xbc, 1, d_xbc, DC, h),
              "conv1d_update")

    def ssm(i, h=sh):
        check(binding.ssm_decode_raw(h_states[i % copies].data_ptr(), xbc.data_ptr(), d_xbc,
                                     proj.data_ptr() + e * (d_inner + d_xbc), N_in, a_log.data_ptr(),
                                     d_param.data_ptr(), dt_bias.data_ptr(), y.data_ptr(), d_inner, 1, H, P, S_, G,
                                     1e-9, 1e9, h), "ssm_decode")

    def layer(i, h=sh):
        w, s_ = W(pin, i)
        check(binding.gemv_fused_raw(x.data_ptr(), 0, w_in.data_ptr(), eps, w, s_, 0, proj.data_ptr(),
                                     1, N_in, K_in, h), "gemv_fused")
        conv(i, h)
        ssm(i, h)
        w, s_ = W(pout, i)
        check(binding.gemv_fused_raw(y.data_ptr(), proj.data_ptr(), w_out.data_ptr(), eps, w, s_, x.data_ptr(),
                                     out.data_ptr(), 1, N_out, K_out, h, ld_gate=N_in), "gemv_fused")

    def layer_in_proj_conv(i, h=sh):
        """The same step with the conv fused into in_proj (3 launches); the conv
        outputs overwrite the xBC columns of the in_proj output, where the SSM
        then reads them."""
        w, s_ = W(pin, i)
        check(binding.gemv_in_proj_raw(x.data_ptr(), w_in.data_ptr(), eps, w, s_, c_states[i % copies].data_ptr(),
                                       cw.data_ptr(), cb.data_ptr(), d_inner, d_xbc, DC, proj.data_ptr(), 1, N_in,
                                       K_in, h), "gemv_in_proj")
        check(binding.ssm_decode_raw(h_states[i % copies].data_ptr(), proj.data_ptr() + e * d_inner, N_in,
                                     proj.data_ptr() + e * (d_inner + d_xbc), N_in, a_log.data_ptr(),
                                     d_param.data_ptr(), dt_bias.data_ptr(), y.data_ptr(), d_inner, 1, H, P, S_, G,
                                     1e-9, 1e9, h), "ssm_decode")
        w, s_ = W(pout, i)
        check(binding.gemv_fused_raw(y.data_ptr(), proj.data_ptr(), w_out.data_ptr(), eps, w, s_, x.data_ptr(),
                                     out.data_ptr(), 1, N_out, K_out, h, ld_gate=N_in), "gemv_fused")

    def graph_of_layers():
        """L layer steps (each with its own weight copies and states) captured
        in one HIP graph; returns us per layer step over `reps` replays."""
        side = torch.cuda.Stream(device=device)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(L):
                layer_in_proj_conv(i, side.cuda_stream)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            h = torch.cuda.current_stream(device).cuda_stream
            for i in range(L):
                layer_in_proj_conv(i, h)
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            ev[2 * r].record(stream)
            g.replay()
            ev[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e3 for r in range(reps)]) / L)

    def timed(fn):
        for i in range(L):
            fn(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for r in range(reps):
            ev[2 * r].record(stream)
            for i in range(L):
                fn(r * L + i)
            ev[2 * r + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[2 * r].elapsed_time(ev[2 * r + 1]) * 1e3 for r in range(reps)]) / L)

    t_layer, t_conv, t_ssm = timed(layer), timed(conv), timed(ssm)
    t_layer3 = timed(layer_in_proj_conv)
    t_graph = graph_of_layers()
    b_conv = 2 * d_xbc * DC * 4 + 2 * d_xbc * e + d_xbc * DC * e + d_xbc * e
    b_ssm = 2 * d_inner * S_ * 4 + d_xbc * e + H * e + d_inner * e + 3 * H * 4
    return {"unit": "us per launch (or per layer step)",
            "state_copies_rotated": copies,
            "layer_step": {"us": round(t_layer, 2),
                           "kernels": "in_proj fused norm GEMV, conv1d update, SSM decode, "
                                      "out_proj fused gated norm GEMV + residual"},
            "layer_step_conv_in_in_proj": {"us": round(t_layer3, 2),
                                           "kernels": "in_proj GEMV with its norm and the conv1d update fused, "
                                                      "SSM decode, out_proj fused"},
            "layer_step_hip_graph": {"us": round(t_graph, 2),
                                     "how": f"{L} layer steps (conv in in_proj) captured in one HIP graph, replayed"},
            "conv1d_update": {"us": round(t_conv, 2), "bytes": b_conv, "GB/s": round(b_conv / t_conv / 1e3, 1),
                              "frac": round(b_conv / t_conv / 1e3 / HBM_PEAK_GBS, 4)},
            "ssm_decode": {"us": round(t_ssm, 2), "bytes": b_ssm, "GB/s": round(b_ssm / t_ssm / 1e3, 1),
                           "frac": round(b_ssm / t_ssm / 1e3 / HBM_PEAK_GBS, 4)}}


def cpu_baseline(budget_s: float):
    """Time the CPU oracle on a bounded sample of the same two workloads."""
    import oracle

    cores = oracle.num_threads()
    dec = inputs.WORKLOADS["decode_m1"]
    pre = inputs.WORKLOADS["prefill_1k"]
    # decode: whole M=1 in_proj + out_proj products, repeated within half the budget
    ops = [(inputs.make(p), p) for p in dec]
    t0 = time.perf_counter()
    reps, nbytes = 0, 0
    while True:
        for (A, W, S), p in ops:
            oracle.w8a16(A, W, S)
            nbytes += p.bytes_moved()
        reps += 1
        if time.perf_counter() - t0 > budget_s / 2:
            break
    t_dec = time.perf_counter() - t0
    # prefill: whole output rows of the M=1024 in_proj (each row = N*K MACs)
    (A, W, S), p = inputs.make(pre[0]), pre[0]
    t0 = time.perf_counter()
    rows, flops = 0, 0
    while time.perf_counter() - t0 < budget_s / 2 and rows < p.M:
        take = min(8, p.M - rows)
        mi = np.repeat(np.arange(rows, rows + take), p.N)
        ni = np.tile(np.arange(p.N), take)
        oracle.w8a16_points(A, W, S, mi, ni)
        rows += take
        flops += 2 * take * p.N * p.K
    t_pre = time.perf_counter() - t0
    return {
        "value": round(nbytes / t_dec / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"{reps} whole M=1 decode passes (in_proj + out_proj) in {t_dec:.1f} s",
        "prefill": {"value": round(flops / t_pre / 1e12, 5), "unit": "TFLOP/s",
                    "sample": f"{rows} whole output rows of the M=1024 in_proj in {t_pre:.1f} s"},
        "layer_steps": cpu_baseline_layer_steps(),
    }


def cpu_baseline_layer_steps(budget_s: float = 1.0):
    """The oracle's norms and decode-step updates on the same shapes as
    `layer_ends` / `decode_layer` (one token, hidden 4096; the prefill norm on
    whole rows), each repeated for about budget_s, as us per call (per row
    for the prefill norm)."""
    import oracle

    dims = inputs.MAMBA2_4K
    H, P, S_, G, DC = dims["heads"], dims["head_dim"], dims["state"], dims["groups"], dims["d_conv"]
    d_inner = H * P
    d_xbc = d_inner + 2 * G * S_
    x = inputs.activations(1, 4096, 9301)
    w = inputs.norm_weight(4096, 9302)
    y = inputs.activations(1, d_inner, 9303)
    z = inputs.activations(1, d_inner, 9304)
    w2 = inputs.norm_weight(d_inner, 9305)
    row = inputs.activations(1, d_xbc + H, 9306)
    cw, cb = inputs.conv_params(d_xbc, DC, 9307)
    cstate = inputs.conv_state(1, d_xbc, DC, 9308).astype(np.float64)
    hstate = inputs.ssm_state(1, H, P, S_, 9309).astype(np.float64)
    a_log, d_param, dt_bias = inputs.ssm_params(H, 9310)
    xbc = inputs.activations(1, d_xbc, 9311)

    def per_call(fn):
        n, t0 = 0, time.perf_counter()
        while n == 0 or time.perf_counter() - t0 < budget_s:
            fn()
            n += 1
        return round((time.perf_counter() - t0) / n * 1e6, 1), n

    out = {"unit": "us per call on the host cores (the fp64 oracle as it stands)"}
    for name, fn in (("rmsnorm_1x4096", lambda: oracle.rmsnorm(x, w, inputs.NORM_EPS)),
                     ("gated_rmsnorm_1x8192", lambda: oracle.rmsnorm(y, w2, inputs.NORM_EPS, gate=z)),
                     ("conv1d_update_10240ch", lambda: oracle.conv1d_update(cstate, row, cw, cb)),
                     ("ssm_decode_128x64x128", lambda: oracle.ssm_decode(hstate, xbc, row[:, d_xbc:], a_log,
                                                                         d_param, dt_bias, G))):
        us, n = per_call(fn)
        out[name] = {"us": us, "calls": n}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-few-tokens", action="store_true",
                    help="skip the few-token report (profiler runs: keeps the dispatch order that "
                         "--summarize-trace / --summarize-counters label)")
    ap.add_argument("--no-layer-ends", action="store_true",
                    help="skip the norm prologue / residual epilogue and layer decode-step timings (profiler runs)")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the vendor bf16 GEMM context leg (torch.matmul on the prefill shapes)")
    ap.add_argument("--no-read-floor", action="store_true",
                    help="skip the plain-read floor of the decode weights (profiler runs)")
    ap.add_argument("--no-large-layer", action="store_true",
                    help="skip the hidden-8192 layer's 8192-token GEMMs and M = 1 GEMVs (profiler runs)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time")
    ap.add_argument("--layers", type=int, default=DEFAULT_LAYERS, help="decode layers (weight copies) per step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a plain device copy of 256 MiB (for HBM counter calibration)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-sq", nargs="+", metavar="CSV",
                    help="matrix-core / LDS counter summary of the GEMM launches: the counter_collection.csv of "
                         "each --pmc pass and the kernel_trace.csv of those runs")
    ap.add_argument("--large-layer-only", action="store_true",
                    help="run only the hidden-8192 layer's leg and print it (profiler runs; with --summarize-* "
                         "label dispatches as that leg's)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.layers, large=args.large_layer_only)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, layers=args.layers)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.layers, large=args.large_layer_only)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (HIP device)", file=sys.stderr)
        sys.exit(2)
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    binding.load()
    if args.large_layer_only:
        stream = torch.cuda.current_stream(device)

        def check_large(st, kind):
            if st != binding.OK:
                raise binding.W8A16Error(f"w8a16_{kind}", st)
        print(json.dumps({"large_layer": large_layer_report(device, stream, check_large)}), flush=True)
        return

    dec, pre = inputs.WORKLOADS["decode_m1"], inputs.WORKLOADS["prefill_1k"]
    projs = [Projection(dec[i], pre[i], device) for i in range(2)]
    stream = torch.cuda.current_stream(device)
    sh = stream.cuda_stream
    torch.cuda.synchronize()

    L = args.layers

    def check(st, kind):
        if st != binding.OK:
            raise binding.W8A16Error(f"w8a16_{kind}", st)

    def step(i, ev=None):
        # ev: 5 events -> [decode in_proj x L][decode out_proj x L][prefill in][prefill out]
        mark = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        mark(0)
        for l in range(L):
            check(projs[0].gemv(i * L + l, sh), "gemv")
        mark(1)
        for l in range(L):
            check(projs[1].gemv(i * L + l, sh), "gemv")
        mark(2)
        check(projs[0].gemm(i, sh), "gemm")
        mark(3)
        check(projs[1].gemm(i, sh), "gemm")
        mark(4)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dur = np.array([[ev[j].elapsed_time(ev[j + 1]) * 1e-3 for j in range(4)] for ev in events])
    dur[:, :2] /= L                                  # per GEMV launch
    mean = dur.mean(axis=0)                          # seconds per launch: gemv in, gemv out, gemm in, gemm out
    floor = None if args.no_read_floor else read_floor_report(projs, device, stream, L, check,
                                                              [mean[0] * 1e6, mean[1] * 1e6])
    few = None if args.no_few_tokens else few_token_report(projs, device, stream, L, check)
    large = None if args.no_large_layer else large_layer_report(device, stream, check)
    vendor = None if args.no_vendor else vendor_gemm_report(device, stream)
    ends = None if args.no_layer_ends else layer_ends_report(projs, device, stream, L, check)
    layer = None if args.no_layer_ends else decode_layer_report(projs, device, stream, L, check)

    if args.copy_calibration:
        src = torch.empty(CALIBRATION_BYTES // 4, dtype=torch.float32, device=device)   # read once, written once
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    b_in, b_out = projs[0].p_dec.bytes_moved(), projs[1].p_dec.bytes_moved()
    f_in, f_out = projs[0].p_pre.flops(), projs[1].p_pre.flops()
    gemv_gbs = (b_in + b_out) / (mean[0] + mean[1]) / 1e9
    gemm_tfs = (f_in + f_out) / (mean[2] + mean[3]) / 1e12

    def roof(bound, achieved, peak, unit, traffic):
        return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic}

    def pair_traffic(kind):
        t = [measured_traffic(kind, f"{kind}_{p}") for p in ("in_proj", "out_proj")]
        return None if None in t else sum(t)

    launches = {
        "gemv_in_proj": roof("hbm", b_in / mean[0] / 1e9, HBM_PEAK_GBS, "GB/s", measured_traffic("gemv", "gemv_in_proj")),
        "gemv_out_proj": roof("hbm", b_out / mean[1] / 1e9, HBM_PEAK_GBS, "GB/s",
                              measured_traffic("gemv", "gemv_out_proj")),
        "gemm_in_proj": roof("mfma", f_in / mean[2] / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s",
                             measured_traffic("gemm", "gemm_in_proj")),
        "gemm_out_proj": roof("mfma", f_out / mean[3] / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s",
                              measured_traffic("gemm", "gemm_out_proj")),
    }
    for k, i in zip(LAUNCHES, range(4)):
        launches[k]["us"] = round(mean[i] * 1e6, 3)
    rec = {
        "metric": METRIC,
        "value": round(gemv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x e4m3 -> fp32 accumulate -> bf16",
        "data": "synthetic (seeded N(0,1) activations; N(0,0.02) weights quantized per 128x128 block to E4M3 + BF16 scales)",
        "config": {
            "workload": "decode_m1 + prefill_1k: Mamba-2 (hidden 4096) in_proj K=4096 N=18560 and "
                        "out_proj K=8192 N=4096; decode GEMV M=1, prefill GEMM M=1024",
            "decode_layers_per_step": L,
            "weight_copies_rotated": [p.copies for p in projs],
            "timing": "HIP events on the launch stream; GEMVs timed over L back-to-back launches",
        },
        "frac_of_hbm_peak": round(gemv_gbs / HBM_PEAK_GBS, 4),
        "kernel_us": {"gemv_in_proj": round(mean[0] * 1e6, 3), "gemv_out_proj": round(mean[1] * 1e6, 3),
                      "gemm_in_proj": round(mean[2] * 1e6, 3), "gemm_out_proj": round(mean[3] * 1e6, 3)},
        # the pair of decode GEMV launches the metric is quoted on (in_proj + out_proj)
        "roofline": roof("hbm", gemv_gbs, HBM_PEAK_GBS, "GB/s", pair_traffic("gemv")),
        "prefill": {
            "value": round(gemm_tfs, 2), "unit": "TFLOP/s",
            "frac_of_mfma_peak": round(gemm_tfs / BF16_PEAK_TFLOPS, 4),
            "roofline": roof("mfma", gemm_tfs, BF16_PEAK_TFLOPS, "TFLOP/s", pair_traffic("gemm")),
        },
        "launches": launches,
        "read_floor": floor,
        "large_layer": large,
        "vendor_bf16_gemm": vendor,
        "few_tokens": few,
        "layer_ends": ends,
        "decode_layer": layer,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(args.cpu_budget),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
