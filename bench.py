"""Throughput of the ModernBERT-base encoder forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu-baseline]
                    [--no-extra]

A step is one whole forward of the 22-layer encoder over one batch of synthetic input already
resident in HBM. The headline (`value`) is workload 4, the largest bf16 batch: 64 packed
sequences with lengths log-uniform in [32, 2048] (28,186 real tokens), random-init weights,
pack meta -> embedding + LN -> 22 layers -> final LN + pooling, replayed as one captured HIP
graph on one stream; the eager rate is reported beside it. The other workloads (3 layers in
fp32 on 300 tokens, the padded batch of 8, one 8192-token sequence, 32 x 8192 tokens in fp16)
are measured the same way, each
in a child process of its own (so that a kernel profile of this process holds the headline's
launches only), and reported under `other_workloads`. Prints one JSON line.

Per-kernel roofline: every launch of the dominant kernel (the kind with the largest share of
one eager forward) is bracketed with HIP events on the stream it runs on, over the eager timed
steps; achieved = algorithmic flops (or bytes) per launch / mean launch duration.
`reference_rates` (outside every timed region): a 1 GiB streaming copy, the library's MFMA-only
calibration kernel (`mbert_mfma_probe`) and PyTorch's GEMM on the projection shapes, the
practical ceilings the fractions can be read against; `roofline.measured_peak` is the copy's
or the probe's rate for the dominant kernel's bound.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "encoded tokens/s, 22L ModernBERT-base bf16 fwd; % bf16 MFMA peak"
PEAK_MFMA_16BIT = 2500.0    # TFLOP/s, dense bf16/fp16 MFMA, MI355X
PEAK_MFMA_F32 = 157.3       # TFLOP/s
PEAK_HBM = 8000.0           # GB/s
CALIB_BYTES = 256 << 20     # streaming calibration kernel: reads and writes this many bytes
CALIB_NAME = "neg_kernel"
XCDS = 8                    # accelerator complex dies, each with its own L2 and GRBM
D, QKV, FF = 768, 2304, 1152
GEMM_FLOPS_PER_TOKEN_LAYER = 2 * (D * QKV + D * D + D * 2 * FF + FF * D)  # 10,027,008


def attention_pairs(lengths, is_global, W=64):
    """In-band (query, key) pairs of one layer: sum L^2 globally, the +-W band locally."""
    tot = 0
    for L in lengths:
        L = int(L)
        if is_global:
            tot += L * L
        else:
            i = np.arange(L)
            tot += int((np.minimum(L - 1, i + W) - np.maximum(0, i - W) + 1).sum())
    return tot


def mfma_flops(kind, T, lengths):
    """Algorithmic matrix flops of one launch of a kernel kind (0 for the row kernels): the
    GEMM's 2 M N K, or 4 * 64 flops per in-band (query, key) pair and head of attention."""
    return {"qkv_rope": 2.0 * T * D * QKV, "wi_geglu": 2.0 * T * D * 2 * FF,
            "wo_resid": 2.0 * T * D * D, "wo2_resid": 2.0 * T * FF * D,
            "attn_global": 4.0 * 64 * 12 * attention_pairs(lengths, True),
            "attn_local": 4.0 * 64 * 12 * attention_pairs(lengths, False)}.get(kind, 0.0)


def kernel_work(kind, T, lengths, dtype_bytes, n_layers=22, n_global=8):
    """(bound, algorithmic work per launch, unit) for a kernel kind of one forward."""
    ds = dtype_bytes
    if kind == "qkv_rope":
        return "mfma", 2.0 * T * D * QKV, "TFLOP/s"
    if kind == "wi_geglu":
        return "mfma", 2.0 * T * D * 2 * FF, "TFLOP/s"
    if kind == "attn_global":
        return "mfma", 4.0 * 64 * 12 * attention_pairs(lengths, True), "TFLOP/s"
    if kind == "attn_local":
        return "hbm", float(T * (QKV * ds + D * ds)), "GB/s"
    if kind == "wo_resid":
        return "hbm", float(T * D * ds + D * D * ds + 2 * T * D * 4), "GB/s"
    if kind == "wo2_resid":
        return "hbm", float(T * FF * ds + D * FF * ds + 2 * T * D * 4), "GB/s"
    if kind == "layernorm":
        return "hbm", float(T * (D * 4 + D * ds) + D * ds), "GB/s"
    if kind == "embed_ln":
        return "hbm", float(T * (4 + D * ds + D * 4 + D * ds) + D * ds), "GB/s"
    if kind == "final_pool":
        return "hbm", float(T * D * 8 + D * ds), "GB/s"
    return "hbm", float(T * 16), "GB/s"


def source_hash() -> str:
    """Hash of the kernel sources and the build script (whose flags shape the kernels)."""
    h = hashlib.sha256()
    pkg = ROOT / "transformer_encoder_amd"
    for p in [*sorted((pkg / "csrc").glob("*")), pkg / "build.py"]:
        h.update(p.name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_kind: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken
    on the current kernel sources; else None."""
    f = ROOT / "profiles" / f"traffic_{kernel_kind}_{workload}.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    if d.get("source_hash") != source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


GEMM_EPI = {"qkv_rope": 1, "wo_resid": 2, "wo2_resid": 2, "wi_geglu": 3}
SUMMARY_DIR = str(ROOT / "profiles")  # where the profile summaries are written
ROW_KERNELS = {"layernorm": "layernorm_kernel", "embed_ln": "embed_ln_kernel",
               "final_pool": "final_ln_kernel"}


def kernel_matches(kind: str, name: str) -> bool:
    """Whether a kernel symbol from a trace belongs to a kernel kind of the forward."""
    import re
    if kind in GEMM_EPI:
        if "gemm_kernel" not in name:
            return False
        ints = [int(x) for x in re.findall(r"Li(\d+)E", name)]  # mangled
        if not ints:  # demangled: gemm_kernel<type, BM, BN, NWM, NWN, EPI, ...>
            m = re.search(r"gemm_kernel<([^>]*)>", name)
            if m:
                ints = [int(x) for x in m.group(1).split(",")[1:] if x.strip().lstrip("-").isdigit()]
        return len(ints) >= 5 and ints[4] == GEMM_EPI[kind]
    if kind in ROW_KERNELS:
        return ROW_KERNELS[kind] in name
    return False


def traffic_summary(fetch_dir: str, write_dir: str, kind: str, workload: str, commands: list):
    """HBM bytes per launch of `kind` from two rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), each scaled by the factor that makes the same counter read
    CALIB_BYTES for the streaming calibration kernel of the same run."""
    import csv
    import glob

    def per_dispatch(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        rows = sorted(csv.DictReader(open(f[0])), key=lambda r: int(r["Dispatch_Id"]))
        # kinds that share a kernel symbol (the two residual GEMMs, global and local
        # attention) are told apart by their order within each forward
        disp = []
        for r in rows:
            if not disp or disp[-1][0] != r["Dispatch_Id"]:
                disp.append((r["Dispatch_Id"], r["Kernel_Name"]))
        kinds = dict(zip([x[0] for x in disp], classify_dispatches([x[1] for x in disp])))
        k_vals, c_vals = [], []
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if kinds.get(r["Dispatch_Id"]) == kind:
                k_vals.append(v)
            elif CALIB_NAME in r["Kernel_Name"]:
                c_vals.append(v)
        if not k_vals or not c_vals:
            raise SystemExit(f"{counter}: kernel or calibration dispatches missing in {d}")
        return sum(k_vals) / len(k_vals), sum(c_vals) / len(c_vals), len(k_vals)

    fk, fc, n_f = per_dispatch(fetch_dir, "FETCH_SIZE")
    wk, wc, n_w = per_dispatch(write_dir, "WRITE_SIZE")
    f_scale = (CALIB_BYTES / 1024.0) / fc
    w_scale = (CALIB_BYTES / 1024.0) / wc
    total = (fk * f_scale + wk * w_scale) * 1024.0
    out = {"kernel_kind": kind, "workload": workload, "source_hash": source_hash(),
           "fetch_kib_per_launch_raw": fk, "write_kib_per_launch_raw": wk,
           "calib_fetch_kib_raw": fc, "calib_write_kib_raw": wc,
           "fetch_scale": f_scale, "write_scale": w_scale, "dispatches": [n_f, n_w],
           "hbm_bytes_per_launch": total, "commands": commands}
    base = Path(SUMMARY_DIR) / f"traffic_{kind}_{workload}"
    base.with_suffix(".json").write_text(json.dumps(out, indent=1) + "\n")
    md = [f"# HBM traffic per launch: {kind}, workload {workload}", "",
          "Counter runs (from the repository root on one MI355X):", "", "```", *commands, "```",
          "", f"- FETCH_SIZE per {kind} launch: {fk:.1f} KiB (raw), calibration kernel "
          f"({CALIB_BYTES >> 20} MiB read + written): {fc:.1f} KiB -> scale {f_scale:.4f}",
          f"- WRITE_SIZE per launch: {wk:.1f} KiB (raw), calibration: {wc:.1f} KiB -> scale "
          f"{w_scale:.4f}",
          f"- HBM bytes per launch (scaled): {total / 1e6:.3f} MB over {n_f} / {n_w} dispatches",
          f"- kernel sources hash: {out['source_hash']}"]
    base.with_suffix(".md").write_text("\n".join(md) + "\n")
    print(json.dumps(out))


def classify_dispatches(names):
    """Kernel kind of every dispatch of a trace, in dispatch order. The two residual GEMMs
    share one symbol (attention Wo, then the MLP Wo in every layer) and so do the two
    attention kinds (global on layers 0, 3, 6, ...): they are told apart by their order
    within each forward, which starts at an embedding launch."""
    kinds, n_res, n_att = [], 0, 0
    for name in names:
        kind = None
        if "embed_ln_kernel" in name:
            kind, n_res, n_att = "embed_ln", 0, 0
        elif "attn_kernel" in name:
            kind = "attn_global" if n_att % 3 == 0 else "attn_local"
            n_att += 1
        elif kernel_matches("wo_resid", name):
            kind = "wo_resid" if n_res % 2 == 0 else "wo2_resid"
            n_res += 1
        else:
            for k in ("qkv_rope", "wi_geglu", "layernorm", "final_pool"):
                if kernel_matches(k, name):
                    kind = k
        kinds.append(kind)
    return kinds


def _trace_rows(directory: str, pattern: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", pattern), recursive=True))
    return [(f, list(csv.DictReader(open(f)))) for f in files]


def profile_summary(trace_dir: str, wid: int, commands: list):
    """profiles/kernel_stats_<workload>.md from a rocprofv3 --kernel-trace --stats run with
    CSV output: per kernel kind of the workload's process (children of the default command
    write their own files), launches, mean duration and the achieved fraction of the
    roofline bound, from the same algorithmic work as the bench line's roofline."""
    from workloads import WORKLOADS, make_batch
    wl = WORKLOADS[wid]
    b = make_batch(wl)
    T, lengths = int(b["cu_seqlens"][-1]), b["lengths"]
    ds = 4 if wl.dtype == "f32" else 2
    slots = int(b["mask"].size) if wl.layout == "padded" else T
    best = None
    # the embedding launch covers 8 rows per workgroup of 256 threads
    full_grid = ((slots + 7) // 8) * 256
    for f, rows in _trace_rows(trace_dir, "*kernel_trace.csv"):
        emb = [r for r in rows if "embed_ln_kernel" in r["Kernel_Name"]]
        if emb and int(emb[0]["Grid_Size_X"]) == full_grid:
            best = (f, rows)
    if best is None:
        raise SystemExit(f"no trace of workload {wl.name} under {trace_dir}")
    f, rows = best
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    # classify each stream's dispatches in its own order (the concurrency legs interleave
    # forwards of several streams)
    kinds = [None] * len(rows)
    by_stream = {}
    for i, r in enumerate(rows):
        by_stream.setdefault(r.get("Stream_Id", "0"), []).append(i)
    for idx in by_stream.values():
        for i, k in zip(idx, classify_dispatches([rows[i]["Kernel_Name"] for i in idx])):
            kinds[i] = k
    # a launch counts when no other kernel was in flight at any time during it: launches that
    # overlapped (the multi-stream legs) share the chip, so their durations are not its own
    start = [int(r["Start_Timestamp"]) for r in rows]
    end = [int(r["End_Timestamp"]) for r in rows]
    order = sorted(range(len(rows)), key=lambda i: start[i])
    alone = [False] * len(rows)
    run_end = -1
    for j, i in enumerate(order):
        nxt = start[order[j + 1]] if j + 1 < len(order) else None
        alone[i] = start[i] >= run_end and (nxt is None or end[i] <= nxt)
        run_end = max(run_end, end[i])
    # whole-batch launches only: a forward's launches count when its embedding launch covered
    # the whole batch (the batch-size sweep's forwards on fewer sequences do not; a persistent
    # GEMM's grid is one workgroup per CU whatever the batch, so its grid does not tell), and
    # of those the largest grid each kind was launched with (the grouped forward's per-group
    # launches have smaller grids)
    names = [k if k is not None else "other: " + r["Kernel_Name"].split("(")[0][:60]
             for r, k in zip(rows, kinds)]
    grid = [int(r.get("Grid_Size_X", 0) or 0) for r in rows]
    in_full = [False] * len(rows)
    for idx in by_stream.values():
        cur = False
        for i in idx:
            if kinds[i] == "embed_ln":
                cur = grid[i] == full_grid
            in_full[i] = cur
    whole = [names[i].startswith("other") or in_full[i] for i in range(len(rows))]
    gmax = {}
    for i, k in enumerate(names):
        if alone[i] and whole[i]:
            gmax[k] = max(gmax.get(k, 0), grid[i])
    per, total_ns, n_over, n_part = {}, 0.0, {}, 0
    for i, k in enumerate(names):
        d = float(end[i] - start[i])
        if not alone[i]:
            n_over[k] = n_over.get(k, 0) + 1
            continue
        if not whole[i] or grid[i] != gmax[k]:
            n_part += 1
            continue
        total_ns += d
        per.setdefault(k, []).append(d)
    md = [f"# Kernel times, workload {wl.name} ({wl.description}; {T} real tokens)", "",
          "Command (from the repository root on one MI355X; the summary is written by "
          "`bench.py --profile-summary`):", "", "```", *commands, "```", "",
          f"Trace file: `{os.path.relpath(f, ROOT)}` (the process of this workload). Launches "
          "that overlapped another kernel in time (the multi-stream legs: "
          f"{sum(n_over.values())} launches) and launches on part of the batch (forwards whose "
          "embedding launch did not cover the whole batch, as the batch-size sweep's, and "
          "launches with a smaller grid than the kind's largest, as the grouped forward's "
          f"per-group launches: {n_part}) are left out; every other launch of the process is "
          "counted.", "",
          "| kernel kind | launches | mean us | total ms | share % | bound | achieved | of peak |",
          "|---|---:|---:|---:|---:|---|---:|---:|"]
    for k, ds_ in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        mean_us = sum(ds_) / len(ds_) / 1e3
        ach = ""
        if not k.startswith("other"):
            bound, work, unit = kernel_work(k, T, lengths, ds)
            if bound == "mfma":
                a = work / (mean_us * 1e-6) / 1e12
                pk = PEAK_MFMA_F32 if wl.dtype == "f32" else PEAK_MFMA_16BIT
                ach = f"| mfma | {a:.0f} TFLOP/s | {a / pk:.3f}"
            else:
                a = work / (mean_us * 1e-6) / 1e9
                ach = f"| hbm | {a:.0f} GB/s | {a / PEAK_HBM:.3f}"
        else:
            ach = "| | |"
        md.append(f"| {k} | {len(ds_)} | {mean_us:.2f} | {sum(ds_) / 1e6:.3f} | "
                  f"{100 * sum(ds_) / total_ns:.2f} {ach} |")
    md += ["", "Achieved = the algorithmic work of one launch (bench.py `kernel_work`) / the mean "
           "launch duration; peaks 2500 TFLOP/s (16-bit MFMA), 157.3 TFLOP/s (fp32 MFMA), "
           "8000 GB/s (HBM)."]
    out = Path(SUMMARY_DIR) / f"kernel_stats_{wl.name}.md"
    out.write_text("\n".join(md) + "\n")
    print(out)


def counter_summary(dirs: list, wid: int, commands: list):
    """profiles/counters_<workload>.md from rocprofv3 --pmc runs (one counter set per run):
    per kernel kind, the mean per dispatch of every counter collected, and the derived MFMA
    busy fraction, non-MFMA VALU instructions per MFMA, L2 hit rate and HBM bytes (FETCH_SIZE
    and WRITE_SIZE scaled by what they read for the streaming calibration kernel)."""
    from workloads import WORKLOADS, make_batch
    wl = WORKLOADS[wid]
    b = make_batch(wl)
    T, lengths = int(b["cu_seqlens"][-1]), b["lengths"]
    flops_per_mfma = 4096.0 if wl.dtype == "f32" else 32768.0  # 32x32x2 f32 / 32x32x16 16-bit
    vals = {}  # kind -> counter -> list
    calib = {}
    for d in dirs:
        for f, rows in _trace_rows(d, "*counter_collection.csv"):
            rows.sort(key=lambda r: int(r["Dispatch_Id"]))
            # one row per (dispatch, counter): classify the dispatches in order
            disp = []
            for r in rows:
                if not disp or disp[-1][0] != r["Dispatch_Id"]:
                    disp.append((r["Dispatch_Id"], r["Kernel_Name"]))
            kinds = dict(zip([x[0] for x in disp], classify_dispatches([x[1] for x in disp])))
            for r in rows:
                c, v = r["Counter_Name"], float(r["Counter_Value"])
                if CALIB_NAME in r["Kernel_Name"]:
                    calib.setdefault(c, []).append(v)
                k = kinds.get(r["Dispatch_Id"])
                if k:
                    vals.setdefault(k, {}).setdefault(c, []).append(v)
    mean = lambda x: sum(x) / len(x)
    simd = 256 * 4  # SIMDs on the chip
    md = [f"# Counters per kernel kind, workload {wl.name}", "",
          "Commands (from the repository root on one MI355X, one counter set per run; the "
          "summary is written by `bench.py --counter-summary`):", "", "```", *commands, "```", "",
          "Per dispatch means. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 "
          "SIMDs) (GRBM_GUI_ACTIVE is summed over the 8 XCDs, each with its own GPU busy counter); VALU/MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA; L2 hit = TCC_HIT / "
          "(TCC_HIT + TCC_MISS); MFMA work = SQ_INSTS_MFMA x the flops of one instruction / the "
          "launch's algorithmic matrix flops (above 1: tile padding and masked key tiles); "
          "HBM MB = FETCH_SIZE and WRITE_SIZE (KiB) scaled by the factor "
          f"that makes each read {CALIB_BYTES >> 20} MiB for the streaming calibration kernel "
          "(`torch.neg` on 256 MiB).", ""]
    fs = ws = None
    if calib.get("FETCH_SIZE"):
        fs = (CALIB_BYTES / 1024.0) / mean(calib["FETCH_SIZE"])
    if calib.get("WRITE_SIZE"):
        ws = (CALIB_BYTES / 1024.0) / mean(calib["WRITE_SIZE"])
    md.append(f"Calibration: FETCH scale {fs if fs is None else round(fs, 4)}, "
              f"WRITE scale {ws if ws is None else round(ws, 4)}.")
    md += ["", "| kernel kind | dispatches | MFMA busy | VALU/MFMA | MFMA work executed / algorithmic | L2 hit | HBM read MB | HBM write MB | raw means |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---|"]
    for k, cs in sorted(vals.items()):
        n = max(len(v) for v in cs.values())
        g = lambda c: mean(cs[c]) if c in cs else None
        busy = (f"{g('SQ_VALU_MFMA_BUSY_CYCLES') / (g('GRBM_GUI_ACTIVE') / XCDS * simd):.3f}"
                if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None and g("GRBM_GUI_ACTIVE") else "")
        vpm = (f"{(g('SQ_INSTS_VALU') - g('SQ_INSTS_MFMA')) / g('SQ_INSTS_MFMA'):.2f}"
               if g("SQ_INSTS_VALU") is not None and g("SQ_INSTS_MFMA") else "")
        hit = (f"{g('TCC_HIT_sum') / (g('TCC_HIT_sum') + g('TCC_MISS_sum')):.3f}"
               if g("TCC_HIT_sum") is not None and g("TCC_MISS_sum") is not None else "")
        rd = f"{g('FETCH_SIZE') * fs * 1024 / 1e6:.1f}" if g("FETCH_SIZE") is not None and fs else ""
        wr = f"{g('WRITE_SIZE') * ws * 1024 / 1e6:.1f}" if g("WRITE_SIZE") is not None and ws else ""
        alg = mfma_flops(k, T, lengths)
        ex = (f"{g('SQ_INSTS_MFMA') * flops_per_mfma / alg:.3f}"
              if g("SQ_INSTS_MFMA") is not None and alg > 0 else "")
        raw = "; ".join(f"{c} {mean(v):.4g}" for c, v in sorted(cs.items()))
        md.append(f"| {k} | {n} | {busy} | {vpm} | {ex} | {hit} | {rd} | {wr} | {raw} |")
    out = Path(SUMMARY_DIR) / f"counters_{wl.name}.md"
    out.write_text("\n".join(md) + "\n")
    print(out)


def cpu_baseline(wl, weights, batch, budget_s=12.0):
    """The oracle as it is, on the host cores: whole sequences of the same workload, in order
    and in repeated passes, until about `budget_s` seconds of CPU work have been spent."""
    from oracle import mbert_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cfg = O.Config(n_layers=wl.n_layers)
    cu = batch["cu_seqlens"]
    S = len(cu) - 1
    done_tok, t_used, seqs = 0, 0.0, 0
    while t_used < budget_s:
        s = seqs % S
        a, b = int(cu[s]), int(cu[s + 1])
        t0 = time.perf_counter()
        O.encode(batch["ids"][a:b], [0, b - a], weights, cfg)
        t_used += time.perf_counter() - t0
        done_tok += b - a
        seqs += 1
    return {"value": round(done_tok / t_used, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{seqs} sequences ({done_tok} tokens; {seqs / S:.2f} passes over the "
                      f"{S} sequences) of the same workload through the float64 numpy oracle, "
                      f"{t_used:.1f} s"}


def measure_heads(B, m, wl, ws, rows_ptr, total_max, T, S, stream, steps):
    """Pooling and the two heads on the forward's own output rows, outside the timed forward
    (kgptalkie, "The Masked-LM Head", "How Do We Put a Classifier on Top?"; candding, "Pooling
    and normalization"): the masked-LM head over every real position, CLS and mean pooling,
    and the 4-label classifier head on mean pooling. `rows_ptr` is the packed fp32 output
    [T, 768]; the workspace still holds the meta buffer. Each is timed with HIP events on the
    stream, averaged over `steps` calls."""
    import torch
    from workloads import Dims, make_head_weights
    from transformer_encoder_amd.model import to_device
    dt = B.DTYPES[wl.dtype]
    hw = make_head_weights(Dims(n_layers=wl.n_layers), wl.dtype, wl.id)
    w = {k: to_device(v, wl.dtype, "cuda") for k, v in hw.items()}
    L = m.layout(total_max, S)
    meta, parts = ws.data_ptr() + L.meta, ws.data_ptr() + L.partials
    vocab = int(m.cfg.vocab)
    hws_n = B.mbert_head_workspace_bytes(dt, T)
    hws = torch.empty(hws_n, dtype=torch.uint8, device="cuda")
    logits = torch.empty((T, vocab), dtype=torch.float32, device="cuda")
    pooled = torch.empty((S, D), dtype=torch.float32, device="cuda")
    cls_logits = torch.empty((S, 4), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    calls = {
        "mlm_head_all_positions": lambda: B.mbert_mlm_head(
            dt, rows_ptr, T, None, T, w["dense"], w["norm"], 1e-5, m.tok_emb, w["decoder_bias"],
            vocab, hws, hws_n, logits, stream),
        "pool_cls_l2": lambda: B.mbert_pool(rows_ptr, total_max, meta, S, B.POOL_CLS | B.POOL_L2,
                                            pooled, parts, stream),
        "pool_mean": lambda: B.mbert_pool(rows_ptr, total_max, meta, S, B.POOL_MEAN, pooled, parts,
                                          stream),
        "classifier_head_4_labels": lambda: B.mbert_classifier_head(
            dt, pooled, S, w["dense"], w["norm"], 1e-5, w["cls_W"], w["cls_b"], 4, hws, hws_n,
            cls_logits, stream),
    }
    res = {"rows": T, "vocab": vocab}
    for name, fn in calls.items():
        fn()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        stream.synchronize()
        res[name] = {"ms": round(e0.elapsed_time(e1) / steps, 5)}
    mlm = res["mlm_head_all_positions"]
    flops = 2.0 * T * D * (D + vocab)
    mlm["algorithmic_tflop"] = round(flops / 1e12, 4)
    mlm["tflops"] = round(flops / (mlm["ms"] * 1e-3) / 1e12, 1)
    mlm["mfma_peak_frac"] = round(flops / (mlm["ms"] * 1e-3) / 1e12 / PEAK_MFMA_16BIT, 4) \
        if wl.dtype != "f32" else None
    mlm["logits_write_gb_s"] = round(T * vocab * 4 / (mlm["ms"] * 1e-3) / 1e9, 1)
    return res


def measure_reference_rates(T: int, dtype: str):
    """Rates of plain library work on the same GPU, outside every timed region: a streaming
    copy (the practical ceiling of the HBM-bound kernels, which read and write once) and
    PyTorch's GEMM (hipBLASLt / rocBLAS) on the forward's four projection shapes with no
    epilogue, as a vendor-library reference for the MFMA-bound ones."""
    import torch
    dev = torch.device("cuda", 0)
    res = {}
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * 4 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    res["hbm_copy_gb_s"] = round(gbs, 1)
    res["hbm_copy_frac_of_peak"] = round(gbs / PEAK_HBM, 4)
    del src, dst
    # the library's MFMA-only calibration kernel: 1024 workgroups of 4 waves (4 per SIMD)
    from transformer_encoder_amd import binding as B
    blocks, iters = 1024, 2000
    probe_out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    for _ in range(2):
        B.mbert_mfma_probe(B.DTYPES[dtype], blocks, iters, probe_out)
    e0.record()
    for _ in range(5):
        B.mbert_mfma_probe(B.DTYPES[dtype], blocks, iters, probe_out)
    e1.record()
    torch.cuda.synchronize()
    flops = blocks * 4 * iters * 4 * (16384.0 if dtype == "f32" else 32768.0)  # per slot
    tf = flops / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e12
    peak = PEAK_MFMA_F32 if dtype == "f32" else PEAK_MFMA_16BIT
    res["mfma_probe_tflops"] = round(tf, 1)
    res["mfma_probe_frac_of_peak"] = round(tf / peak, 4)
    del probe_out
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    gemms = {}
    peak = PEAK_MFMA_F32 if dtype == "f32" else PEAK_MFMA_16BIT
    for name, (K, N) in {"qkv_wi": (768, 2304), "wo": (768, 768), "wo2": (1152, 768)}.items():
        a = torch.randn(T, K, device=dev).to(tdt)
        b = torch.randn(K, N, device=dev).to(tdt)  # [K, N] row-major
        w = torch.randn(N, K, device=dev).to(tdt)  # [N, K]: a Linear weight, as the kernels here
        best = None
        # 2-D products only: a @ b, and F.linear (a @ w^T, the layout of the forward's weights)
        for layout, fn in (("a@b", lambda: torch.mm(a, b)),
                           ("linear(a,w)", lambda: torch.nn.functional.linear(a, w))):
            for _ in range(3):
                fn()
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / 20 * 1e3
            if best is None or us < best[0]:
                best = (us, layout)
        us, layout = best
        tf = 2.0 * T * K * N / (us * 1e-6) / 1e12
        gemms[f"{name}_{T}x{K}x{N}"] = {"us": round(us, 2), "tflops": round(tf, 1),
                                        "frac_of_peak": round(tf / peak, 4), "faster_layout": layout}
        del a, b, w
    res["torch_plain_gemm"] = gemms
    return res


def measure_sweep(B, m, batch, steps_small=10, steps_large=3):
    """Throughput against batch size for a packed batch of equal-length sequences: the first
    n sequences for n = 1, 2, 4, ... up to all of them, each forward captured as one graph
    and replayed (tokens/s at every residency up to the full batch)."""
    import torch
    dev = torch.device("cuda", 0)
    lengths = np.asarray(batch["lengths"])
    cu_all = np.asarray(batch["cu_seqlens"])
    res = {}
    n = 1
    while n <= len(lengths):
        T = int(cu_all[n])
        ids = torch.from_numpy(np.ascontiguousarray(batch["ids"][:T].astype(np.int32))).to(dev)
        cu = torch.from_numpy(np.ascontiguousarray(cu_all[:n + 1].astype(np.int32))).to(dev)
        ws = m.workspace(T, n)
        out = torch.empty((T, D), dtype=torch.float32, device=dev)
        pooled = torch.empty((n, D), dtype=torch.float32, device=dev)
        st = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            g = B.mbert_graph_capture(m.w, ids, cu, n, T, ws, ws.numel(), out, pooled, st)
        steps = steps_small if n <= 8 else steps_large
        for _ in range(2):
            B.mbert_graph_launch(g, st)
        st.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            B.mbert_graph_launch(g, st)
        e1.record(st)
        st.synchronize()
        ms = e0.elapsed_time(e1) / steps
        B.mbert_graph_destroy(g)
        res[str(n)] = {"tokens": T, "ms_per_step": round(ms, 4), "steps": steps,
                       "tokens_per_s": round(T / (ms * 1e-3), 1)}
        del ids, cu, ws, out, pooled
        n *= 2
    return res


def measure_concurrency(B, m, padded, args_in, out_like, pooled_like, ws_like, steps, warmup):
    """Throughput with G independent batches in flight on G streams (one captured forward per
    stream, each with its own workspace and outputs, launched round-robin): the rate a server
    sees when requests overlap. Reported beside the single-stream value, never as it."""
    import torch
    res = {}
    for G in (2, 4):
        streams = [torch.cuda.Stream() for _ in range(G)]
        graphs, keep = [], []
        for st in streams:
            with torch.cuda.stream(st):
                ws = torch.empty_like(ws_like)
                o = torch.empty_like(out_like)
                p = torch.empty_like(pooled_like)
                keep += [ws, o, p]
                if padded:
                    ids_pad, mask, Bn, Tp = args_in
                    g = B.mbert_graph_capture_padded(m.w, ids_pad, mask, Bn, Tp, ws, ws.numel(), o, p, st)
                else:
                    ids, cu, S, T = args_in
                    g = B.mbert_graph_capture(m.w, ids, cu, S, T, ws, ws.numel(), o, p, st)
            graphs.append(g)
        for i in range(warmup * G):
            B.mbert_graph_launch(graphs[i % G], streams[i % G])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            B.mbert_graph_launch(graphs[i % G], streams[i % G])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        for g in graphs:
            B.mbert_graph_destroy(g)
        res[str(G)] = {"ms_per_step": round(dt * 1e3 / steps, 4), "steps": steps}
        del keep
    return res


def measure_grouped(B, m, ids_pad, mask, Bn, Tp, out_ref, pooled_ref, steps, warmup):
    """One batch's forward split into G groups of whole sequences on G streams (one captured
    graph with a branch per group): time per forward and whether it equals the single-stream
    forward bit for bit."""
    import torch
    res = {}
    for G in (2, 4, 8):
        streams = [torch.cuda.Stream() for _ in range(G - 1)]
        main_s = torch.cuda.Stream()
        nbytes = B.mbert_workspace_bytes_grouped(m.cfg, m.dtype, Bn, Tp, G)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        o = torch.empty_like(out_ref)
        p = torch.empty_like(pooled_ref)
        g = B.mbert_graph_capture_padded_grouped(m.w, ids_pad, mask, Bn, Tp, G, ws, nbytes, o, p,
                                                 streams, main_s)
        for _ in range(warmup):
            B.mbert_graph_launch(g, main_s)
        main_s.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main_s)
        for _ in range(steps):
            B.mbert_graph_launch(g, main_s)
        e1.record(main_s)
        main_s.synchronize()
        ms = e0.elapsed_time(e1) / steps
        B.mbert_graph_destroy(g)
        res[str(G)] = {"graph_ms_per_step": round(ms, 4),
                       "equal_to_single_stream": bool(torch.equal(o, out_ref) and torch.equal(p, pooled_ref))}
        del ws, o, p
    return res


# steps / warmup of the other workloads' runs (about 150 ms per forward for 262,144 tokens)
EXTRA_RUNS = {1: (100, 10), 2: (100, 10), 3: (50, 5), 5: (10, 2), 4: (50, 5)}


def other_workloads(headline: int) -> dict:
    """The other workloads, each measured by this script in a child process of its own (graph
    replay, dominant-kernel roofline and reference rates, no CPU baseline or head timings),
    keyed by name."""
    import subprocess
    from workloads import WORKLOADS
    res = {}
    for wid in (1, 2, 3, 5, 4):
        if wid == headline:
            continue
        steps, warmup = EXTRA_RUNS[wid]
        cmd = [sys.executable, str(Path(__file__).resolve()), "--workload", str(wid),
               "--steps", str(steps), "--warmup", str(warmup), "--no-cpu-baseline",
               "--no-heads", "--no-extra"]
        print(f"bench: workload {wid} ({WORKLOADS[wid].name}) in a child process", file=sys.stderr,
              flush=True)
        proc = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=600)
        lines = [ln for ln in proc.stdout.splitlines() if ln.startswith("{")]
        if proc.returncode != 0 or not lines:
            res[WORKLOADS[wid].name] = {"error": f"exit status {proc.returncode}"}
            continue
        d = json.loads(lines[-1])
        keep = ("value", "unit", "ms_per_step", "steps", "warmup", "dtype", "mfma_peak_frac",
                "algorithmic_tflop_per_step", "eager_ms_per_step", "graph_ms_per_step",
                "single_stream_graph_ms_per_step", "graph_matches_eager", "roofline",
                "kernel_ms_share", "reference_rates", "batch_sweep")
        res[WORKLOADS[wid].name] = {"config": d["config"], **{k: d[k] for k in keep if k in d}}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip workload 5's throughput sweep over 1, 2, 4, ... 32 sequences")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the streaming-copy and library-GEMM reference rates")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --workload, not the other workloads in child processes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of the graph")
    ap.add_argument("--no-heads", action="store_true", help="skip the pooling and head timings")
    ap.add_argument("--groups", type=int, default=3,
                    help="padded workloads: time the forward with the batch split into this many "
                         "groups of whole sequences on as many streams (1 = one stream)")
    ap.add_argument("--no-fold", action="store_true",
                    help="run the LayerNorms as separate kernels instead of folding them into the GEMMs")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<kind>_<workload>.{json,md} from two "
                         "rocprofv3 --pmc runs of this script and exit")
    ap.add_argument("--kind", default="wi_geglu", help="kernel kind for --traffic-summary")
    ap.add_argument("--profile-summary", metavar="TRACE_DIR",
                    help="write profiles/kernel_stats_<workload>.md from a rocprofv3 "
                         "--kernel-trace --stats --output-format csv run and exit")
    ap.add_argument("--summary-dir", help="directory for the summaries (default profiles/)")
    ap.add_argument("--counter-summary", nargs="+", metavar="PMC_DIR",
                    help="write profiles/counters_<workload>.md from rocprofv3 --pmc runs and exit")
    ap.add_argument("--command", action="append", default=[],
                    help="the counter-run commands, recorded in the summary")
    args = ap.parse_args()
    global SUMMARY_DIR
    if args.summary_dir:
        SUMMARY_DIR = args.summary_dir
        os.makedirs(SUMMARY_DIR, exist_ok=True)
    if args.profile_summary:
        profile_summary(args.profile_summary, args.workload, args.command)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.workload, args.command)
        return
    if args.traffic_summary:
        from workloads import WORKLOADS
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.kind,
                        WORKLOADS[args.workload].name, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch

    from transformer_encoder_amd import binding as B
    from transformer_encoder_amd.model import DeviceModel, int32_device
    from workloads import WORKLOADS, make_batch, workload_weights

    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload]
    weights = workload_weights(wl.id)
    batch = make_batch(wl)
    lengths = batch["lengths"]
    T = int(batch["cu_seqlens"][-1])
    S = len(lengths)
    m = DeviceModel(weights, wl.dtype, fold=not args.no_fold)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream()
    padded = wl.layout == "padded"
    with torch.cuda.stream(stream):
        if padded:
            ids_pad, mask = int32_device(batch["ids_pad"], dev), int32_device(batch["mask"], dev)
            Bn, Tp = batch["mask"].shape
            ws = m.workspace(Bn * Tp, Bn)
            out = torch.empty((Bn, Tp, D), dtype=torch.float32, device=dev)
        else:
            ids, cu = int32_device(batch["ids"], dev), int32_device(batch["cu_seqlens"], dev)
            ws = m.workspace(T, S)
            out = torch.empty((T, D), dtype=torch.float32, device=dev)
        pooled = torch.empty((S, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def eager(kind=None, timer=None):
        if padded:
            if timer is None:
                B.mbert_encode_padded(m.w, ids_pad, mask, Bn, Tp, ws, ws.numel(), out, pooled, stream)
            else:
                B.mbert_encode_padded_timed(m.w, ids_pad, mask, Bn, Tp, ws, ws.numel(), out, pooled,
                                            kind, timer, stream)
        else:
            if timer is None:
                B.mbert_encode(m.w, ids, cu, S, T, ws, ws.numel(), out, pooled, stream)
            else:
                B.mbert_encode_timed(m.w, ids, cu, S, T, ws, ws.numel(), out, pooled, kind, timer,
                                     stream)

    max_launches = max(64, 64 * (args.steps + 2))
    timer = B.mbert_timer_create(max_launches)
    # ---- which kernel kind dominates one eager forward
    for _ in range(max(1, args.warmup)):
        eager()
    stream.synchronize()
    share = {}
    for name, kind in B.KERNEL_KINDS.items():
        B.mbert_timer_reset(timer)
        eager(kind, timer)
        n, ms = B.mbert_timer_read(timer)
        share[name] = ms
    dominant = max(share, key=share.get)
    dom_kind = B.KERNEL_KINDS[dominant]

    # ---- eager timed region (events around every dominant-kernel launch)
    B.mbert_timer_reset(timer)
    t0e, t1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream.synchronize()
    t0e.record(stream)
    for _ in range(args.steps):
        eager(dom_kind, timer)
    t1e.record(stream)
    stream.synchronize()
    eager_ms = t0e.elapsed_time(t1e) / args.steps
    n_launch, dom_ms_total = B.mbert_timer_read(timer)
    dom_avg_ms = dom_ms_total / max(n_launch, 1)

    # ---- graph-replayed timed region
    gws = torch.empty_like(ws)
    gout = torch.empty_like(out)
    gpool = torch.empty_like(pooled)
    def time_graph(g, s):
        for _ in range(args.warmup):
            B.mbert_graph_launch(g, s)
        s.synchronize()
        t0g, t1g = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0g.record(s)
        for _ in range(args.steps):
            B.mbert_graph_launch(g, s)
        t1g.record(s)
        s.synchronize()
        return t0g.elapsed_time(t1g) / args.steps

    with torch.cuda.stream(stream):
        if padded:
            g = B.mbert_graph_capture_padded(m.w, ids_pad, mask, Bn, Tp, gws, gws.numel(), gout,
                                             gpool, stream)
        else:
            g = B.mbert_graph_capture(m.w, ids, cu, S, T, gws, gws.numel(), gout, gpool, stream)
    single_ms = time_graph(g, stream)
    same = bool(torch.equal(gout, out) and torch.equal(gpool, pooled))
    B.mbert_graph_destroy(g)
    B.mbert_timer_destroy(timer)
    # the timed forward: one batch split into `groups` groups of whole sequences, each group's
    # forward on its own stream in one captured graph. Its outputs are bitwise those of the
    # same grouped forward run eagerly; against the one-stream forward they agree within
    # rounding (a group's attention grid is small enough for the split-key kernel).
    groups = args.groups if (padded and args.groups > 1) else 1
    graph_ms = single_ms
    grouped_diff = None
    if groups > 1:
        xstreams = [torch.cuda.Stream() for _ in range(groups - 1)]
        nb = B.mbert_workspace_bytes_grouped(m.cfg, m.dtype, Bn, Tp, groups)
        gws2 = torch.empty(nb, dtype=torch.uint8, device=dev)
        eout, epool = torch.empty_like(out), torch.empty_like(pooled)
        B.mbert_encode_padded_grouped(m.w, ids_pad, mask, Bn, Tp, groups, gws2, nb, eout, epool,
                                      xstreams, stream)
        stream.synchronize()
        grouped_diff = float((eout - out).abs().max())
        gout.zero_()
        gpool.zero_()
        torch.cuda.synchronize()
        g = B.mbert_graph_capture_padded_grouped(m.w, ids_pad, mask, Bn, Tp, groups, gws2, nb,
                                                 gout, gpool, xstreams, stream)
        graph_ms = time_graph(g, stream)
        same = same and bool(torch.equal(gout, eout) and torch.equal(gpool, epool))
        B.mbert_graph_destroy(g)
        del gws2

    # a plain streaming kernel of known size (reads and writes CALIB_BYTES), outside the timed
    # region: rocprofv3 counter runs scale FETCH_SIZE / WRITE_SIZE by what they read for it
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    torch.neg(calib_src, out=calib_dst)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    grouped = None
    if padded and not args.no_heads:
        grouped = measure_grouped(B, m, ids_pad, mask, Bn, Tp, out, pooled, args.steps, args.warmup)
        for v in grouped.values():
            v["tokens_per_s"] = round(T / (v["graph_ms_per_step"] * 1e-3), 1)

    concurrency = None
    if not args.no_heads:
        cargs = (ids_pad, mask, Bn, Tp) if padded else (ids, cu, S, T)
        concurrency = measure_concurrency(B, m, padded, cargs, out, pooled, ws, args.steps,
                                          args.warmup)
        for v in concurrency.values():
            v["tokens_per_s"] = round(T / (v["ms_per_step"] * 1e-3), 1)

    sweep = None
    if wl.id == 5 and not args.no_sweep:
        sweep = measure_sweep(B, m, batch)

    reference_rates = None
    if not args.no_reference:
        reference_rates = measure_reference_rates(T, wl.dtype)

    keymask = None
    if padded and not args.no_heads:
        # the same padded batch run at full width with a key padding mask (no unpadding)
        kws = torch.empty_like(ws)
        kout = torch.empty_like(out)
        kpool = torch.empty_like(pooled)
        kfn = lambda: B.mbert_encode_padded_keymask(m.w, ids_pad, mask, Bn, Tp, kws, kws.numel(),
                                                    kout, kpool, stream)
        kfn()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(min(args.steps, 20)):
            kfn()
        e1.record(stream)
        stream.synchronize()
        kms = e0.elapsed_time(e1) / min(args.steps, 20)
        real = torch.from_numpy(batch["mask"].astype(bool)).to(dev)
        keymask = {"eager_ms_per_step": round(kms, 4), "tokens_per_s": round(T / (kms * 1e-3), 1),
                   "rows_computed": Bn * Tp,
                   "real_rows_equal_unpadded": bool(torch.equal(kout[real], out[real]))}
        del kws, kout, kpool

    heads = None
    if not args.no_heads:
        # the last eager forward's rows, packed (input set-up for the head timings: the real
        # rows of the padded output gathered in order, or the packed batch's output as is)
        total_max = Bn * Tp if padded else T
        if padded:
            packed_rows = torch.zeros((total_max, 768), dtype=torch.float32, device=dev)
            packed_rows[:T] = out.view(-1, 768)[torch.from_numpy(batch["mask"].astype(bool).ravel()).to(dev)]
            rows_ptr = packed_rows.data_ptr()
        else:
            rows_ptr = out.data_ptr()
        heads = measure_heads(B, m, wl, ws, rows_ptr, total_max, T, S, stream,
                              min(args.steps, 20))

    ms = eager_ms if args.eager else graph_ms
    tokens_per_s = T / (ms * 1e-3)
    pairs_g = attention_pairs(lengths, True)
    pairs_l = attention_pairs(lengths, False)
    n_layers = wl.n_layers
    n_glob = len([i for i in range(n_layers) if i % 3 == 0])
    flops = (GEMM_FLOPS_PER_TOKEN_LAYER * T * n_layers
             + 3072.0 * (pairs_g * n_glob + pairs_l * (n_layers - n_glob)))
    peak_mfma = PEAK_MFMA_F32 if wl.dtype == "f32" else PEAK_MFMA_16BIT
    ds = 4 if wl.dtype == "f32" else 2
    bound, work, unit = kernel_work(dominant, T, lengths, ds)
    if bound == "mfma":
        achieved = work / (dom_avg_ms * 1e-3) / 1e12
        peak = peak_mfma
    else:
        achieved = work / (dom_avg_ms * 1e-3) / 1e9
        peak = PEAK_HBM
    traffic = traffic_from_profiles(dominant, wl.name)
    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded uniform token ids, random-init N(0,0.02) weights)",
        "config": {"workload": wl.name, "description": wl.description, "real_tokens": T,
                   "sequences": S, "padded_to": wl.pad_to, "layers": n_layers,
                   "layernorms": "folded into the GEMMs" if m.folded is not None else "separate kernels",
                   "streams": 1 if args.eager else groups,
                   "timed": "eager launches" if args.eager else (
                       "HIP graph replay" if groups == 1 else
                       f"HIP graph replay, the batch split into {groups} groups of whole sequences "
                       f"on {groups} streams (outputs bitwise equal to the eager grouped forward, within "
                       f"rounding of one stream)")},
        "mfma_peak_frac": round(flops / (ms * 1e-3) / 1e12 / peak_mfma, 4),
        "algorithmic_tflop_per_step": round(flops / 1e12, 4),
        "eager_ms_per_step": round(eager_ms, 4),
        "single_stream_graph_ms_per_step": round(single_ms, 4),
        "graph_ms_per_step": round(graph_ms, 4),
        "graph_matches_eager": same,
        "grouped_vs_one_stream_max_abs": None if grouped_diff is None else float(f"{grouped_diff:.3e}"),
        "kernel_ms_share": {k: round(v, 4) for k, v in sorted(share.items(), key=lambda x: -x[1])},
        "roofline": {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "launches_timed": n_launch,
                     "avg_launch_ms": round(dom_avg_ms, 5),
                     "work_per_launch": work},
    }
    if grouped is not None:
        line["grouped_streams"] = grouped
    if concurrency is not None:
        line["concurrent_streams"] = concurrency
    if keymask is not None:
        line["padded_keymask"] = keymask
    if heads is not None:
        line["heads"] = heads
    if sweep is not None:
        line["batch_sweep"] = sweep
    if reference_rates is not None:
        line["reference_rates"] = reference_rates
        measured = (reference_rates["mfma_probe_tflops"] if bound == "mfma"
                    else reference_rates["hbm_copy_gb_s"])
        line["roofline"]["measured_peak"] = measured
        line["roofline"]["frac_of_measured_peak"] = round(achieved / measured, 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, weights, batch)
    if not args.no_extra:
        del m, ws, gws, gout, gpool, out, pooled
        torch.cuda.empty_cache()
        line["other_workloads"] = other_workloads(wl.id)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
