"""Benchmark of the FLASH layer forward (GAU with mixed chunk attention) on one
MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--copy-calibration]
    python bench.py --summarize-stats STATS_CSV --command CMD --out FILE.md
    python bench.py --summarize-traffic FETCH_CSV WRITE_CSV --command CMD
    python bench.py --decode | --backward | --sweep | --vendor-gemm

A step is one full forward of the layer (all six kernels) over one batch of
seeded synthetic input, B=2 sequences of T=8192 tokens, d=768, e=1536, s=128,
chunk C=256, bf16 storage with fp32 accumulation, causal.  Inputs are resident
in HBM before the timed region starts.  Prints one JSON line.

The timed region is K plain gau_forward calls between two synchronisations.
Just before it, loops of whole forwards and of forwards without the dominant
kernel (the projection GEMM), each loop between two HIP events on the stream
the kernels run on, give that kernel's average duration inside a forward; the
roofline object is its algorithmic FLOPs per launch divided by that duration,
against the dense bf16 MFMA peak.  Per-stage times (kernels_us)
come from another pass with events around every stage.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4 SIMDs x 1024 dense bf16 FLOP/clk x 2.4 GHz
PEAK_FP32_TFLOPS = 157.3    # dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "GAU/FLASH layer fwd tokens/sec at d=768 T=8192 C=256; % bf16 MFMA peak"
STAGES = ["proj", "chunk_scores", "chunk_state", "chunk_scan", "chunk_attn", "out_gemm"]
DOMINANT = "proj"
DOM_BATCH = 20  # back-to-back launches of the dominant kernel between two events
DOM_REPS = 5    # loops per measurement of the dominant kernel (median)


def algorithmic_flops(B, T, d, e, s, C, causal=True):
    """Algorithmic FLOPs of one layer forward, per stage.

    Dense GEMMs count 2 FLOP per multiply-add.  The intra-chunk score and value
    products count the causal lower triangle with its diagonal, C(C+1)/2 pairs
    per chunk (the full C^2 when non-causal)."""
    M = B * T
    pairs = C * (C + 1) / 2 if causal else C * C
    G = T // C
    return {
        "proj": 2.0 * M * d * (2 * e + s),
        "chunk_scores": 2.0 * B * G * pairs * s,
        "chunk_state": 2.0 * M * s * e,
        "chunk_scan": 0.0,
        "chunk_attn": 2.0 * B * G * pairs * e + 2.0 * M * s * e,
        "out_gemm": 2.0 * M * e * d,
    }


def algorithmic_bytes(B, T, d, e, s, C, causal=True, eb=2):
    """Minimum HBM bytes each stage must move with this decomposition."""
    M = B * T
    G = T // C
    Gp = G if causal else 1
    st = B * G * e * s
    pairs = C * (C + 1) // 2 if causal else C * C
    return {
        "proj": M * d * eb + (2 * e + s) * d * eb + 2 * M * e * eb + 4 * M * s * eb,
        "chunk_scores": 2 * M * s * eb + B * G * pairs * eb,
        "chunk_state": M * (e + s) * eb + st * eb,
        "chunk_scan": st * eb + B * Gp * e * s * eb,
        "chunk_attn": B * G * pairs * eb + M * (s + 2 * e) * eb + B * Gp * e * s * eb + M * e * eb,
        "out_gemm": M * e * eb + e * d * eb + M * d * eb,
    }


SOURCES = {"proj": "proj_gemm"}


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def source_hash(name):
    """Hash of the code (comments and blank lines dropped) of a kernel's
    source file and the device headers it includes."""
    csrc = os.path.join(ROOT, "chunked_linear_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in (SOURCES.get(name, name) + ".hip", "gemm_core.h", "gau_device.h"):
        with open(os.path.join(csrc, f)) as fh:
            code = _COMMENTS.sub("", fh.read())
        h.update("\n".join(l.rstrip() for l in code.splitlines() if l.strip()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None if there is none or the kernel source has changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_B2_T8192_d768_C256_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo) and its logical CPU count."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name} ({os.cpu_count()} logical CPUs, {len(os.sched_getaffinity(0))} usable)"


def cpu_baseline(cfg, inp, min_s=12.0, max_passes=100):
    """The float64 oracle, as it stands, on the host cores: whole sequences of
    the timed workload, one after another, repeated until at least min_s of
    CPU work has been timed."""
    from oracle import gau_oracle as orc
    done, t0 = 0, time.perf_counter()
    while True:
        b = done % cfg["B"]
        orc.flash_forward(inp["X"][b:b + 1], inp["W_u"], inp["W_v"], inp["W_z"], inp["W_o"], inp["gamma"],
                          inp["beta"], inp["relpos"], cfg["C"], cfg["causal"])
        done += 1
        dt = time.perf_counter() - t0
        if (dt >= min_s and done % cfg["B"] == 0) or done >= max_passes * cfg["B"]:
            break
    return {"value": done * cfg["T"] / dt, "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{done} sequences of T={cfg['T']} ({done // cfg['B']} passes over the B={cfg['B']} "
                      f"timed workload), float64 numpy, {dt:.1f} s"}


# Size of the calibration copy (bytes read = bytes written).
COPY_BYTES = 256 << 20
PROFILE_TAG = "B2_T8192_d768_C256"


def mfma_probe(torch, g, blocks=1024, iters=1000, reps=5):
    """The bf16 MFMA rate the chip sustains with operands in registers
    (gau_probe_mfma): median over reps launches, each timed with HIP events.
    Outside the timed region; the layer is also quoted against it."""
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    g.probe_mfma(blocks, iters, out)  # warm-up
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        flops = g.probe_mfma(blocks, iters, out)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    t = float(np.median(times))
    return {"tflops": flops / t / 1e12, "frac_of_published": flops / t / 1e12 / PEAK_BF16_TFLOPS,
            "flops_per_launch": flops, "ms": t * 1e3, "blocks": blocks, "iters": iters}


def vendor_gemm():
    """The plain bf16 GEMMs of the layer's two dense contractions through
    torch (its vendor BLAS), no epilogue: a yardstick for the projection and
    output kernels, which also apply SiLU, the heads, the transposed V store
    or the residual.  One JSON line per shape; not part of the layer path."""
    import torch

    torch.manual_seed(0)
    shapes = [("proj d768 e1536 (X [W_u|W_v|W_z])", 16384, 3200, 768),
              ("proj without W_z", 16384, 3072, 768),
              ("out d768 e1536 (Y W_o)", 16384, 768, 1536),
              ("proj d1024 e2048", 16384, 4224, 1024),
              ("out d1024 e2048", 16384, 1024, 2048)]
    for name, M, N, K in shapes:
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
        for _ in range(10):
            c = a @ b.t()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(50):
                c = a @ b.t()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / 50)
        us = float(np.median(times))
        print(json.dumps({"vendor_gemm": name, "M": M, "N": N, "K": K, "us": us,
                          "tflops": 2.0 * M * N * K / us / 1e6}), flush=True)
        del a, b, c


def copy_calibration(torch):
    """Three plain device-to-device copies of COPY_BYTES (torch's copy_ of a
    contiguous tensor runs the HIP runtime's copyBuffer blit kernel): the HBM
    counters of a kernel whose traffic is known exactly."""
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def _short(name):
    n = name.replace("void gau::(anonymous namespace)::", "").replace("gau::(anonymous namespace)::", "")
    return n.split("(")[0]


def summarize_stats(csv_path, command, out, title=None):
    """Markdown summary of a rocprofv3 --stats kernel table."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    title = title or "FLASH layer forward, B=2 T=8192 d=768 e=1536 s=128 C=256, bf16, causal"
    lines = [f"# rocprofv3 kernel statistics: {title}", "", "Command (from the repository root, one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


FORWARD_KERNELS = ["proj_kernel", "chunk_scores_state_kernel", "chunk_scan_kernel", "chunk_attn_kernel",
                   "out_gemm_kernel"]


def summarize_forward_trace(trace_csv, command, out, title=None):
    """Markdown summary of the plain forwards in a rocprofv3 kernel trace: the
    runs of the forward's five launches in order, per-kernel duration
    statistics over them and the forward's span (first start to last end)."""
    import csv
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))

    def kind(name):
        for k in FORWARD_KERNELS:
            if k in name:
                return k
        return None

    kinds = [kind(r["Kernel_Name"]) for r in rows]
    fwd = [rows[i:i + 5] for i in range(len(rows) - 4) if kinds[i:i + 5] == FORWARD_KERNELS]
    title = title or "FLASH layer forward, B=2 T=8192 d=768 e=1536 s=128 C=256, bf16, causal"
    span = [(int(f[-1]["End_Timestamp"]) - int(f[0]["Start_Timestamp"])) / 1e3 for f in fwd]
    lines = [f"# rocprofv3 kernel trace, whole forwards: {title}", "", "Command (from the repository root, one MI355X):",
             "", "```", command, "```", "",
             f"{len(fwd)} forwards found (five launches in order); durations from each launch's start to its end.",
             f"Forward span, first start to last end: median {np.median(span):.1f} us, mean {np.mean(span):.1f} us.",
             "", "| kernel | launches | median (us) | mean (us) | min (us) | max (us) | share of span |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for k, name in enumerate(FORWARD_KERNELS):
        d = np.array([(int(f[k]["End_Timestamp"]) - int(f[k]["Start_Timestamp"])) / 1e3 for f in fwd])
        lines.append(f"| `{name}` | {len(d)} | {np.median(d):.1f} | {d.mean():.1f} | {d.min():.1f} | {d.max():.1f} | "
                     f"{100 * np.median(d) / np.median(span):.1f}% |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_rows(csv_path, counter):
    """(kernel name, grid size, value) per dispatch from a rocprofv3 --pmc csv."""
    import csv
    return [(r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]))
            for r in csv.DictReader(open(csv_path)) if r["Counter_Name"] == counter]


def summarize_traffic(fetch_csv, write_csv, command):
    """HBM bytes per launch of the dominant kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the reading of the same
    counter for the calibration copy of COPY_BYTES."""
    out = {}
    for csv_path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        rows = _counter_rows(csv_path, counter)
        blits = [r for r in rows if r[0] == "__amd_rocclr_copyBuffer"]
        big = max(g for _, g, _ in blits) if blits else 0
        copy = [v for _, g, v in blits if g == big]
        dom = [v for k, _, v in rows if f"{DOMINANT}_kernel<gau::bf16" in k]
        if len(copy) != 3 or not dom:
            raise SystemExit(f"{csv_path}: expected 3 calibration copies and {DOMINANT} dispatches")
        kib_copy, kib_dom = sum(copy) / len(copy), sum(dom) / len(dom)
        factor = kib_copy * 1024.0 / COPY_BYTES  # counter bytes per true byte
        out[counter] = {"kib_per_dispatch": kib_dom, "copy_kib_per_dispatch": kib_copy,
                        "scale": factor, "bytes_per_launch": kib_dom * 1024.0 / factor,
                        "dispatches": len(dom)}
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    cfg = dict(B=2, T=8192, d=768, e=1536, s=128, C=256)
    algo = algorithmic_bytes(**cfg)[DOMINANT]
    rec = {"kernel": DOMINANT, "workload": "layer_bf16_" + PROFILE_TAG, "source_sha256_16": source_hash(DOMINANT),
           "hbm_bytes_per_launch": total, "algorithmic_bytes_per_launch": algo, "counters": out,
           "calibration": f"torch device copy of {COPY_BYTES} bytes (read {COPY_BYTES}, write {COPY_BYTES})",
           "command": command}
    base = os.path.join(ROOT, "profiles", f"{DOMINANT}_{PROFILE_TAG}_traffic")
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# HBM traffic of `{DOMINANT}` (projection GEMM: U, V, Z heads), FLASH layer B=2 T=8192 d=768 e=1536 "
             "s=128 C=256, bf16", "", "Commands (from the repository root, one MI355X; one counter per run):",
             "", "```", command, "```", "",
             "| counter | KiB / dispatch | calibration copy KiB / dispatch | scale (counter B per true B) | "
             "bytes / launch |", "|---|---:|---:|---:|---:|"]
    for c, v in out.items():
        lines.append(f"| {c} | {v['kib_per_dispatch']:.0f} | {v['copy_kib_per_dispatch']:.0f} | "
                     f"{v['scale']:.4f} | {v['bytes_per_launch'] / 1e6:.2f} MB |")
    lines += ["", f"Total {total / 1e6:.2f} MB per launch against {algo / 1e6:.2f} MB algorithmic "
              f"(ratio {total / algo:.2f}).", ""]
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(rec))


def summarize_counters(csvs, stats_csv, command, out):
    """Per-kernel table from rocprofv3 --pmc runs of the headline bench: MFMA
    utilisation (MfmaUtil: busy MFMA cycles over active cycles of all SIMDs),
    MFMA FLOPs (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), and HBM bytes (FETCH_SIZE,
    WRITE_SIZE scaled by the calibration copy in the same run), with rates
    over the kernel-trace average durations of stats_csv."""
    import csv
    dur = {_short(r["Name"]): float(r["AverageNs"]) * 1e-9 for r in csv.DictReader(open(stats_csv))}
    vals = {}  # (kernel, counter) -> list of per-dispatch values
    scale = {}
    for path in csvs:
        rows = list(csv.DictReader(open(path)))
        for counter in sorted({r["Counter_Name"] for r in rows}):
            crow = _counter_rows(path, counter)
            if counter in ("FETCH_SIZE", "WRITE_SIZE"):
                blits = [r for r in crow if r[0] == "__amd_rocclr_copyBuffer"]
                big = max(g for _, g, _ in blits) if blits else 0
                copy = [v for _, g, v in blits if g == big]
                if len(copy) != 3:
                    raise SystemExit(f"{path}: expected 3 calibration copies")
                scale[counter] = sum(copy) / 3 * 1024.0 / COPY_BYTES
            for k, _, v in crow:
                if "gau::" not in k:  # the calibration copy and torch's input set-up
                    continue
                vals.setdefault((_short(k), counter), []).append(v)
    kernels = sorted({k for k, _ in vals}, key=lambda k: -dur.get(k, 0))
    mean = lambda k, c: (sum(vals[(k, c)]) / len(vals[(k, c)])) if (k, c) in vals else None
    lines = ["# Hardware counters per kernel: FLASH layer forward, B=2 T=8192 d=768 e=1536 s=128 C=256, bf16, causal",
             "", "Commands (from the repository root, one MI355X; one counter group per run):", "", "```", command,
             "```", "",
             "MFMA util = MfmaUtil (busy MFMA cycles summed over SIMDs / (active GPU cycles x SIMDs)); MFMA "
             "TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP / trace duration; HBM MB = FETCH_SIZE and "
             "WRITE_SIZE per dispatch divided by each counter's reading per true byte of a 256 MiB device copy "
             + ", ".join(f"({c}: {v:.4f})" for c, v in sorted(scale.items())) + "; GB/s over the trace duration.",
             "LDS read B/clk/CU = SQ_INSTS_LDS_LOAD_BANDWIDTH x 64 B / (GRBM_GUI_ACTIVE / 8 x 256 CUs) (the "
             "reported GRBM_GUI_ACTIVE is the sum over the 8 XCDs); bank conflict = SQ_LDS_BANK_CONFLICT / "
             "SQ_LDS_IDX_ACTIVE (share of the LDS's busy cycles stalled by bank conflicts); LDS busy = "
             "SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / 8 x 256 CUs).",
             "", "| kernel | trace avg (us) | MFMA util | MFMA TFLOP/s | HBM read MB | HBM write MB | HBM GB/s | "
             "LDS read B/clk/CU | LDS bank conflict | LDS busy |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for k in kernels:
        t = dur.get(k)
        util = mean(k, "MfmaUtil")
        mops = mean(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        rd = mean(k, "FETCH_SIZE")
        wr = mean(k, "WRITE_SIZE")
        rd = rd * 1024.0 / scale["FETCH_SIZE"] if rd is not None else None
        wr = wr * 1024.0 / scale["WRITE_SIZE"] if wr is not None else None
        f = lambda x, fmt: (fmt % x) if x is not None else "-"
        tf = mops * 512 / t / 1e12 if (mops is not None and t) else None
        gbs = (rd + wr) / t / 1e9 if (rd is not None and wr is not None and t) else None
        gui, idx = mean(k, "GRBM_GUI_ACTIVE"), mean(k, "SQ_LDS_IDX_ACTIVE")
        ldsb, conf = mean(k, "SQ_INSTS_LDS_LOAD_BANDWIDTH"), mean(k, "SQ_LDS_BANK_CONFLICT")
        cu_clk = gui / 8 * 256 if gui else None
        ld_rate = ldsb * 64 / cu_clk if (ldsb is not None and cu_clk) else None
        cshare = conf / idx if (conf is not None and idx) else None
        busy = idx / cu_clk if (idx is not None and cu_clk) else None
        lines.append(f"| `{k}` | {f(t * 1e6 if t else None, '%.1f')} | {f(util, '%.1f%%')} | {f(tf, '%.0f')} | "
                     f"{f(rd / 1e6 if rd is not None else None, '%.1f')} | "
                     f"{f(wr / 1e6 if wr is not None else None, '%.1f')} | {f(gbs, '%.0f')} | "
                     f"{f(ld_rate, '%.1f')} | {f(100 * cshare if cshare is not None else None, '%.1f%%')} | "
                     f"{f(100 * busy if busy is not None else None, '%.1f%%')} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def sweep(steps, warmup):
    """Forward throughput of every named workload (single layers causal and
    not, C = 256 and 512, the 24-layer stack), one single-call forward per
    step, inputs resident in HBM.  One JSON line per workload; not the
    headline line."""
    import torch
    import chunked_linear_attention_amd as g
    from chunked_linear_attention_amd import inputs

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    for name, wl in inputs.WORKLOADS.items():
        B, T, d, e, s, C = (wl[k] for k in ("B", "T", "d", "e", "s", "C"))
        causal = wl["causal"]
        bf = wl["dtype"] == "bf16"
        tdt = torch.bfloat16 if bf else torch.float32
        gc = g.make_config(B, T, d, e, s, C, causal, g.GAU_BF16 if bf else g.GAU_F32, rope=wl.get("rope", False))
        layer_flops = sum(algorithmic_flops(B, T, d, e, s, C, causal).values())
        if "layers" in wl:
            X, layers = inputs.make_stack_inputs(**wl)
            dev = [g.device_layer(L, tdt) for L in layers]
            x0 = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).cuda()
            x = x0.clone()
            ws = torch.empty(g.stack_workspace_bytes(gc), dtype=torch.uint8, device="cuda")
            n_layers = len(layers)

            def fwd():
                x.copy_(x0)  # the residual stream is updated in place
                g.stack_forward(gc, x, dev, ws, stream=stream)
        else:
            inp = inputs.make_layer_inputs(**wl)
            dev = g.device_layer(inp, tdt)
            ws = torch.empty(g.workspace_bytes(gc), dtype=torch.uint8, device="cuda")
            O = torch.empty((B, T, d), dtype=tdt, device="cuda")
            args_l = (dev["X"], dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"], dev["offset"],
                      dev["relpos"], O, ws)
            n_layers = 1

            def fwd():
                g.forward(gc, *args_l, stream=stream)
        for _ in range(warmup):
            fwd()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fwd()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        flops = layer_flops * n_layers
        peak = PEAK_BF16_TFLOPS if bf else PEAK_FP32_TFLOPS
        print(json.dumps({"sweep": name, "tokens_per_s": B * T / sec, "ms_per_forward": sec * 1e3,
                          "layers": n_layers, "tflops": flops / sec / 1e12,
                          "frac_of_peak": flops / sec / 1e12 / peak,
                          "peak": f"{'bf16' if bf else 'fp32'} {peak} TFLOP/s",
                          "note": "stack: includes the copy that restores the input" if n_layers > 1 else ""}),
              flush=True)
        del dev, ws
        torch.cuda.empty_cache()


def decode_bytes(B, d, e, s, C, eb=2):
    """Algorithmic HBM bytes of one decoding step averaged over a chunk: every
    weight once, and per sequence the state P as the steps read it (its copy in
    the element type), the chunk cache rows read so far (on average (C+1)/2
    slots) and the step's own rows written."""
    weights = (2 * e + s) * d * eb + e * d * eb
    per_seq = s * e * eb + (C + 1) / 2 * (e + s) * eb + (e + 2 * s) * eb + 2 * d * eb
    return weights + B * per_seq


DECODE_BATCHES = (1, 2, 8, 32, 128)


def summarize_decode_trace(trace_csv, command, out, steps=256, warmup=20):
    """Markdown table of the decoding kernels per batch size from a rocprofv3
    --kernel-trace of `bench.py --decode` (dispatches in launch order: for each
    batch size, warmup + steps decoding steps)."""
    import csv
    import re
    rows = [r for r in csv.DictReader(open(trace_csv)) if "decode_" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = {}
    idx, cnt = 0, 0
    for r in rows:
        name = re.search(r"(decode_\w+?)(_mfma)?_kernel", r["Kernel_Name"]).group(1)
        if name == "decode_proj":
            cnt += 1
            if cnt > steps + warmup:
                idx, cnt = idx + 1, 1
        per.setdefault((DECODE_BATCHES[idx], name), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    kernels = ["decode_proj", "decode_attn", "decode_out", "decode_state"]
    lines = ["# rocprofv3 kernel trace: incremental decoding, d=768 e=1536 s=128 C=256, bf16", "",
             "Command (from the repository root, one MI355X):", "", "```", command, "```", "",
             "Average duration per launch (us) by batch size B (from B = 9 the projection and output "
             "products are the `_mfma` kernels); decode_state runs once per chunk "
             f"({steps} steps per batch size, {warmup} warm-up steps before them).", "",
             "| B | " + " | ".join(f"`{k}`" for k in kernels) + " |",
             "|---:|" + "---:|" * len(kernels)]
    for B in DECODE_BATCHES:
        cells = []
        for k in kernels:
            v = per.get((B, k), [])
            cells.append(f"{sum(v) / len(v):.1f}" if v else "-")
        lines.append(f"| {B} | " + " | ".join(cells) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def decode_bench(steps, warmup, batches=DECODE_BATCHES):
    """Incremental decoding at the headline layer's shape (d=768, e=1536,
    s=128, C=256, bf16): one JSON line per batch size, timed over `steps`
    consecutive positions (a whole chunk by default, so the state update at
    the chunk's end is included)."""
    import torch
    import chunked_linear_attention_amd as g
    from chunked_linear_attention_amd import inputs

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    wl = inputs.WORKLOADS[inputs.HEADLINE]
    d, e, s, C = (wl[k] for k in ("d", "e", "s", "C"))
    for B in batches:
        inp = inputs.make_layer_inputs(B=B, T=steps + warmup, d=d, e=e, s=s, C=C, seed=wl["seed"])
        dev = g.device_layer(inp, torch.bfloat16)
        T = ((steps + warmup + C - 1) // C) * C
        cfg = g.make_config(B, T, d, e, s, C, True, g.GAU_BF16)
        ws = torch.empty(g.decode_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        xs = [dev["X"][:, t].contiguous() for t in range(steps + warmup)]
        o = torch.empty((B, d), dtype=torch.bfloat16, device="cuda")
        w = (dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"], dev["offset"], dev["relpos"])

        def run(t0, n):
            for t in range(t0, t0 + n):
                g.decode_step(cfg, t % T, xs[t], *w, o, ws, stream=stream)

        g.decode_reset(cfg, ws, stream=stream)
        run(0, warmup)
        g.decode_reset(cfg, ws, stream=stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(0, steps)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        byt = decode_bytes(B, d, e, s, C)
        print(json.dumps({"decode": f"layer_bf16_d{d}_e{e}_s{s}_C{C}", "batch": B, "steps": steps,
                          "us_per_step": sec * 1e6, "tokens_per_s": B / sec,
                          "roofline": {"bound": "hbm", "achieved": byt / sec / 1e9, "peak": PEAK_HBM_GBS,
                                       "unit": "GB/s", "frac": byt / sec / 1e9 / PEAK_HBM_GBS,
                                       "algorithmic_bytes_per_step": byt}}), flush=True)
        del dev, ws, xs
        torch.cuda.empty_cache()


def summarize_backward_trace(trace_csv, command, out):
    """Markdown table of one gau_backward call (the last complete one) from a
    rocprofv3 --kernel-trace of `bench.py --backward`: every launch in order
    with its grid and duration, then the totals per kernel."""
    import csv
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [_short(r["Kernel_Name"]) for r in rows]
    starts = [i for i, n in enumerate(names) if n.startswith("proj_kernel")]
    a, b = starts[-2], starts[-1]   # each call begins with the recompute's projection
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    total = sum(dur(rows[i]) for i in range(a, b))
    wall = (int(rows[b - 1]["End_Timestamp"]) - int(rows[a]["Start_Timestamp"])) / 1e3
    lines = ["# rocprofv3 kernel trace: FLASH layer backward (gau_backward), B=2 T=8192 d=768 e=1536 s=128 "
             "C=256, bf16, causal", "", "Command (from the repository root, one MI355X):", "", "```", command,
             "```", "", f"One call: {b - a} launches, {total:.1f} us of kernel time, {wall:.1f} us from the first "
             "launch's start to the last one's end.", "", "| # | kernel | workgroups | us |", "|---:|---|---:|---:|"]
    per = {}
    for i in range(a, b):
        r = rows[i]
        wg = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0) // max(int(r.get("Workgroup_Size_X", 256) or 256), 1)
        lines.append(f"| {i - a} | `{names[i]}` | {wg} | {dur(r):.1f} |")
        per.setdefault(names[i], []).append(dur(r))
    lines += ["", "| kernel | launches per call | us per call | share |", "|---|---:|---:|---:|"]
    for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{n}` | {len(v)} | {sum(v):.1f} | {100 * sum(v) / total:.1f}% |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def backward_bench(steps, warmup):
    """The layer's backward pass (gau_backward: the forward's intermediates
    recomputed, then every gradient) at the headline workload: one JSON line.
    Algorithmic FLOPs are twice the forward's (each product of the forward has
    two gradient products); the recomputation is not counted."""
    import torch
    import chunked_linear_attention_amd as g
    from chunked_linear_attention_amd import inputs

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    name = inputs.HEADLINE
    wl, inp = inputs.workload_inputs(name)
    B, T, d, e, s, C = (wl[k] for k in ("B", "T", "d", "e", "s", "C"))
    dev = g.device_layer(inp, torch.bfloat16)
    dO = g.device_tensor(inputs.make_output_grad(B, T, d, seed=wl["seed"]), torch.bfloat16)
    cfg = g.make_config(B, T, d, e, s, C, True, g.GAU_BF16)
    ws = torch.empty(g.backward_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    like = {"X": (B, T, d), "W_u": (e, d), "W_v": (e, d), "W_z": (s, d), "W_o": (d, e), "scale": (4, s),
            "offset": (4, s), "relpos": (2 * C - 1,)}
    grads = {k: torch.empty(like[k], dtype=torch.float32, device="cuda") for k in g.GRAD_NAMES}
    w = (dev["X"], dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"], dev["offset"], dev["relpos"])

    def step():
        g.backward(cfg, *w, dO, grads, ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    fl = 2.0 * sum(algorithmic_flops(B, T, d, e, s, C).values())
    print(json.dumps({"backward": name, "steps": steps, "warmup": warmup, "ms_per_step": sec * 1e3,
                      "tokens_per_s": B * T / sec, "workspace_bytes": ws.numel(),
                      "roofline": {"bound": "mfma", "achieved": fl / sec / 1e12, "peak": PEAK_BF16_TFLOPS,
                                   "unit": "TFLOP/s", "frac": fl / sec / 1e12 / PEAK_BF16_TFLOPS,
                                   "algorithmic_flops_per_step": fl}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the measurement, run the copy that calibrates the HBM counters")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV")
    ap.add_argument("--summarize-forward-trace", metavar="TRACE_CSV",
                    help="per-kernel durations over the plain forwards of a rocprofv3 kernel trace")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_CSV",
                    help="per-kernel MFMA utilisation and HBM traffic from rocprofv3 --pmc csv files (needs --stats)")
    ap.add_argument("--stats", metavar="STATS_CSV", help="kernel statistics csv for --summarize-counters")
    ap.add_argument("--command", default="")
    ap.add_argument("--out")
    ap.add_argument("--summarize-decode-trace", metavar="TRACE_CSV")
    ap.add_argument("--summarize-backward-trace", metavar="TRACE_CSV")
    ap.add_argument("--decode", action="store_true",
                    help="incremental decoding throughput per batch size (one JSON line each)")
    ap.add_argument("--backward", action="store_true",
                    help="the layer's backward pass at the headline workload (one JSON line)")
    ap.add_argument("--title", help="heading of a --summarize-stats table")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time torch's plain bf16 GEMMs of the layer's dense shapes (a yardstick, one JSON line each)")
    ap.add_argument("--sweep", action="store_true",
                    help="throughput of every named workload (one JSON line each) instead of the headline line")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.command, args.out, args.title)
        return
    if args.summarize_forward_trace:
        summarize_forward_trace(args.summarize_forward_trace, args.command, args.out, args.title)
        return
    if args.summarize_decode_trace:
        summarize_decode_trace(args.summarize_decode_trace, args.command, args.out)
        return
    if args.summarize_backward_trace:
        summarize_backward_trace(args.summarize_backward_trace, args.command, args.out)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.stats, args.command, args.out)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep(args.steps, args.warmup)
        return
    if args.vendor_gemm:
        vendor_gemm()
        return
    if args.decode:
        decode_bench(args.steps if args.steps != 100 else 256, args.warmup)
        return
    if args.backward:
        backward_bench(args.steps if args.steps != 100 else 20, args.warmup if args.warmup != 20 else 3)
        return

    import torch
    import chunked_linear_attention_amd as g
    from chunked_linear_attention_amd import inputs

    name = inputs.HEADLINE
    cfg, inp = inputs.workload_inputs(name)
    B, T, d, e, s, C = (cfg[k] for k in ("B", "T", "d", "e", "s", "C"))
    causal = cfg["causal"]
    torch.cuda.set_device(0)
    dev = g.device_layer(inp, torch.bfloat16)
    gc = g.make_config(B, T, d, e, s, C, causal, g.GAU_BF16)
    ws = torch.empty(g.workspace_bytes(gc), dtype=torch.uint8, device="cuda")
    O = torch.empty((B, T, d), dtype=torch.bfloat16, device="cuda")
    args_l = (dev["X"], dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"], dev["offset"],
              dev["relpos"], O, ws)
    stream = torch.cuda.current_stream()

    dom = STAGES.index(DOMINANT)

    def step():
        """One forward: one gau_forward call (six kernels) on the stream."""
        g.forward(gc, *args_l, stream=stream)

    def step_bracketed(ev):
        """The same forward as three calls, with the dominant kernel's stage
        alone between the two events ev = (start, end)."""
        if dom > 0:
            g.forward_stages(gc, 0, dom - 1, *args_l, stream=stream)
        ev[0].record(stream)
        g.forward_stages(gc, dom, dom, *args_l, stream=stream)
        ev[1].record(stream)
        if dom + 1 < len(STAGES):
            g.forward_stages(gc, dom + 1, len(STAGES) - 1, *args_l, stream=stream)

    K = args.steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Diagnostics before the timed region (they also settle the clocks):
    # (1) the dominant kernel's duration inside forwards, from HIP events on
    # the stream the kernels run on, one pair around each loop: K whole
    # forwards, then K forwards without the dominant stage (the later stages
    # read the workspace it left), DOM_REPS times each, interleaved; the
    # difference of the medians per forward is that stage's cost in a forward
    # (no event sits between its launch and its neighbours').  (2) the same
    # kernel in batches of DOM_BATCH back-to-back launches between two events
    # (median of DOM_REPS).  (3) the forward split into three calls with
    # events around the dominant kernel, K of them.  (4) every stage alone
    # between events, and scores + states as the forward runs them.
    def loop_ms(first, last, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            g.forward_stages(gc, first, last, *args_l, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    full_ms, rest_ms = [], []
    for _ in range(DOM_REPS):
        full_ms.append(loop_ms(0, len(STAGES) - 1, K))
        rest_ms.append(loop_ms(dom + 1, len(STAGES) - 1, K) if dom == 0 else loop_ms(0, len(STAGES) - 1, K))
    dom_ms = float(np.median(full_ms) - np.median(rest_ms))
    batch_ms = [loop_ms(dom, dom, DOM_BATCH) for _ in range(DOM_REPS)]
    dom_batch_ms = float(np.median(batch_ms))
    dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t_split = time.perf_counter()
    for ev in dom_ev:
        step_bracketed(ev)
    torch.cuda.synchronize()
    split_ms_per_step = (time.perf_counter() - t_split) * 1e3 / K
    dom_in_forward_ms = float(np.mean([a.elapsed_time(b) for a, b in dom_ev]))

    stage_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(K)]
    for k in range(K):
        for i in range(len(STAGES)):
            stage_ev[k][i].record(stream)
            g.forward_stages(gc, i, i, *args_l, stream=stream)
        stage_ev[k][len(STAGES)].record(stream)
    torch.cuda.synchronize()
    per_stage = {n: float(np.mean([stage_ev[k][i].elapsed_time(stage_ev[k][i + 1]) for k in range(K)]))
                 for i, n in enumerate(STAGES)}  # ms
    i_sc = STAGES.index("chunk_scores")
    pair_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in pair_ev:
        a.record(stream)
        g.forward_stages(gc, i_sc, i_sc + 1, *args_l, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    pair_ms = float(np.mean([a.elapsed_time(b) for a, b in pair_ev]))
    for _ in range(args.warmup):
        step()

    # timed region: exactly K plain forwards, a synchronisation on each side
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same loop once more (a repeat of the timed region, reported beside it)
    t1 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall_repeat = time.perf_counter() - t1

    tokens = B * T
    ms_per_step = wall * 1e3 / K
    value = tokens * K / wall
    flops = algorithmic_flops(B, T, d, e, s, C, causal)
    bytes_ = algorithmic_bytes(B, T, d, e, s, C, causal)
    layer_flops = sum(flops.values())
    achieved = flops[DOMINANT] / (dom_ms * 1e-3) / 1e12
    traffic = measured_traffic(DOMINANT)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, random-init weights)",
        "config": {"workload": name, "B": B, "T": T, "d": d, "e": e, "s": s, "C": C,
                   "causal": causal, "global_batch": B, "seq_len": T},
        "layer_frac_of_bf16_peak": layer_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "layer_tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "kernel": DOMINANT, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "algorithmic_flops_per_launch": flops[DOMINANT], "avg_launch_us": dom_ms * 1e3,
                     "event_samples": 2 * DOM_REPS * K,
                     "event_note": f"the kernel's cost inside forwards: median per-forward time of {K} whole "
                                   f"forwards minus that of {K} forwards without its stage, {DOM_REPS} loops each, "
                                   "one pair of HIP events on the launch stream around each loop, just before "
                                   "the timed region",
                     "avg_launch_us_back_to_back": dom_batch_ms * 1e3,
                     "avg_launch_us_in_forward_with_events": dom_in_forward_ms * 1e3},
        "kernels_us": {n: per_stage[n] * 1e3 for n in STAGES},
        "kernels_gbs": {n: bytes_[n] / (per_stage[n] * 1e-3) / 1e9 for n in STAGES},
        "kernels_tflops": {n: flops[n] / (per_stage[n] * 1e-3) / 1e12 for n in STAGES},
        "kernels_us_combined": {"chunk_scores+chunk_state": pair_ms * 1e3},
        "kernels_us_note": "each stage launched alone between two timing events (about 3 us of GPU time "
                           "each); the kernel trace gives the durations inside one forward",
        "ms_per_step_repeat": wall_repeat * 1e3 / K,
        "ms_per_step_split_calls": split_ms_per_step,
    }
    probe = mfma_probe(torch, g)
    out["mfma_probe"] = probe
    out["roofline"]["frac_of_probe"] = achieved / probe["tflops"]
    out["layer_frac_of_probe"] = out["layer_tflops"] / probe["tflops"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        copy_calibration(torch)


if __name__ == "__main__":
    main()
