#!/usr/bin/env python3
"""Benchmark of the Hyper-Connections residual path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the path over one batch of synthetic tokens whose
inputs are already resident in HBM:
  static-bf16   pre (read-mix + RMSNorm) then post (stream-mix + write-back)
                with shared static weights; F is a given tensor (default)
  dynamic-bf16  per-token weights (MFMA projection + tanh), then pre, post
  dynamic-fp8   the same with FP8 E4M3 H, W and F
  mhc-bf16      Sinkhorn records from per-token logits, then pre, post
  chain-bf16    78 layers of pre, tanh block, post (reported, not graded)
  decode-bf16   the same 78-layer loop at 64 tokens in flight (latency-bound;
                use --graph to replay it as one HIP graph)
  static-fp8    static-bf16's step with FP8 E4M3 storage (16384 tokens: the
                same HBM bytes per step)
  tiny-f32      one small fp32 layer

Timing: W untimed steps, then K timed steps between device synchronisations,
with HIP events recorded on the launch stream around every kernel.  Each step
uses the next of several buffer sets whose total size is at least twice the
256 MB Infinity Cache, so that re-reads cannot come from it.  Prints one JSON
line; details go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s + achieved HBM GB/s (% roofline), fused HC pre+post, n=4 d=4096 bf16"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20      # Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")

KERNEL_SOURCES = {
    "pre_mix": "hc_rows.hip", "post_mix": "hc_rows.hip", "post_pre_mix": "hc_rows.hip",
    "block_tanh": "hc_rows.hip", "weights": "hc_weights.hip", "sinkhorn": "hc_weights.hip",
    "post_mix_backward": "hc_backward.hip", "pre_mix_backward": "hc_backward.hip",
    "sum_records": "hc_backward.hip", "weights_backward": "hc_weights_bwd.hip",
    "weights_backward_stream": "hc_weights_bwd.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """A C/HIP source without its comments and blank space: what the
    compiler sees, so an edit to a comment leaves the hash alone."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(" ".join(l.split()) for l in src.splitlines() if l.strip())


def source_sha(kernel: str) -> str:
    """Hash of the code a kernel is built from (its file + the shared device
    header, comments left out), used to invalidate stale counter
    summaries."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "hc_device.h"):
        with open(os.path.join(ROOT, "hyper_connections_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


class Timer:
    """Counts launches per kernel; with `per_kernel`, also records HIP events
    on the launch stream around every launch."""

    def __init__(self, torch, per_kernel: bool):
        self.torch = torch
        self.per_kernel = per_kernel
        self.pairs = {}
        self.counts = {}

    def run(self, name, fn):
        self.counts[name] = self.counts.get(name, 0) + 1
        if not self.per_kernel:
            return fn()
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        r = fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))
        return r

    def avg_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.pairs.items()}

    def clear(self):
        self.pairs = {}
        self.counts = {}


COPY_PROBE_BYTES = 512 * 2 ** 20   # bytes read (and written) by the calibration copy
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense, published
CLOCK_GHZ = 2.4
SIMDS = 1024                       # 256 CUs x 4
XCDS = 8

# kernel name in the traces, where it differs from "<kernel>_kernel<"
KERNEL_TAGS = {"post_mix_backward": "post_bwd_kernel<", "pre_mix_backward": "pre_bwd_kernel<",
               "weights_backward_stream": "wgrad_mfma_kernel<"}


def summarize_mfma(pmc_csv: str, kernel: str, workload: str, cmds: list):
    """Matrix-core use of `kernel` from one rocprofv3 --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_LDS_BANK_CONFLICT,
    SQ_LDS_IDX_ACTIVE and GRBM_GUI_ACTIVE.  Per dispatch: MFMA busy fraction =
    busy SIMD-cycles / (active cycles x 1024 SIMDs), where GRBM_GUI_ACTIVE
    sums the 8 XCDs' active cycles; MFMA flops = MOPS x 512.  Writes
    profiles/<kernel>_<workload>_mfma.{json,md}."""
    import csv
    from collections import defaultdict
    tag = KERNEL_TAGS.get(kernel, f"{kernel}_kernel<")
    per = defaultdict(dict)
    with open(pmc_csv) as fh:
        for r in csv.DictReader(fh):
            if tag in r["Kernel_Name"]:
                per[r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
    need = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT",
            "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE")
    disp = [v for v in per.values() if all(k in v for k in need)]
    if not disp:
        raise SystemExit(f"no {kernel} dispatches with all of {need}")
    mean = lambda k: sum(v[k] for v in disp) / len(disp)  # noqa: E731
    cycles = mean("GRBM_GUI_ACTIVE") / XCDS
    busy = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (cycles * SIMDS)
    flops = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
    secs = cycles / (CLOCK_GHZ * 1e9)
    from hyper_connections_amd import workloads
    wl = workloads.workload(workload)
    if kernel == "weights_backward_stream":
        # two contractions of T x K x d: dhbar = W^T dz and dW = dz hbar^T
        useful = 4.0 * wl.T * wl.K * wl.d
        note = ("Two contractions of 16384 tokens x K x d each (dhbar = W^T dz, dW = sum dz hbar^T), "
                "K = 24 padded to 32.  The split-bf16 operands (hi + lo) make dhbar two products and "
                "dW three, so the matrix cores execute 3.3x the useful flops (five products of "
                "32-row tiles for two contractions of 24 rows).  The pass is "
                "bound by its memory access: a copy of the kernel with both products removed ran at "
                "the same speed.")
    else:
        useful = 2.0 * wl.T * wl.n * wl.K * wl.d
        note = ("The projection is 24 output columns padded to two 16-column MFMA tiles, so the "
                "matrix cores do 32/24 of the useful flops.  The kernel is bound by HBM: its flops per "
                "byte are about 12x below the bf16 MFMA ridge, and the matrix cores idle most of the "
                "time by design.")
    rec = {"kernel": kernel, "workload": workload, "source_sha": source_sha(kernel),
           "dispatches": len(disp), "active_cycles_per_xcd": round(cycles),
           "duration_us_from_cycles": round(secs * 1e6, 2),
           "mfma_busy_fraction": round(busy, 4), "mfma_flops_per_launch": int(flops),
           "useful_flops_per_launch": int(useful),
           "mfma_tflops": round(flops / secs / 1e12, 1),
           "mfma_peak_tflops_bf16": MFMA_PEAK_TFLOPS["bf16"],
           "lds_bank_conflict_over_active": round(mean("SQ_LDS_BANK_CONFLICT") /
                                                  max(mean("SQ_LDS_IDX_ACTIVE"), 1.0), 4),
           "commands": cmds}
    base = os.path.join(PROFILES, f"{kernel}_{workload}_mfma")
    with open(base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(base + ".md", "w") as fh:
        fh.write(f"# Matrix-core use of {kernel}, workload {workload}\n\n")
        fh.write("Command (run as `cd /tmp && export TMPDIR=/tmp` first; paths are relative to the repository root):\n\n")
        for c in cmds:
            fh.write(f"    {c}\n")
        fh.write(f"\nSummarised with `python bench.py --summarize-mfma PMC_CSV --kernel {kernel} "
                 f"--workload {workload}`.\n\n| quantity | value |\n|---|---|\n")
        for k in ("dispatches", "active_cycles_per_xcd", "duration_us_from_cycles", "mfma_busy_fraction",
                  "mfma_flops_per_launch", "useful_flops_per_launch", "mfma_tflops",
                  "mfma_peak_tflops_bf16", "lds_bank_conflict_over_active", "source_sha"):
            fh.write(f"| {k} | {rec[k]} |\n")
        fh.write("\n" + note + "\n")
    log(f"[bench] wrote {base}.json: MFMA busy {busy:.1%}, {flops / secs / 1e12:.1f} TFLOP/s")


def summarize_counters(fetch_csv: str, write_csv: str, kernel: str, workload: str, cmds: list,
                       fold: bool = True):
    """Turn two rocprofv3 --pmc runs of this benchmark (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) into HBM bytes per launch of `kernel`.

    Each counter is scaled by what it reads for the benchmark's calibration
    copy (torch copy_ of COPY_PROBE_BYTES, a blit kernel that reads and writes
    exactly that many bytes).  Writes profiles/<kernel>_<workload>_counters.json
    (read by the benchmark for roofline.traffic) and a .md next to it."""
    import csv

    def rows(path, counter):
        out = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.append(r)
        return out

    fetch, write = rows(fetch_csv, "FETCH_SIZE"), rows(write_csv, "WRITE_SIZE")
    probe_kib = COPY_PROBE_BYTES / 1024
    wprobe = [r for r in write if "copyBuffer" in r["Kernel_Name"]
              and abs(float(r["Counter_Value"]) - probe_kib) < 0.01 * probe_kib]
    ids = {r["Dispatch_Id"] for r in wprobe}
    fprobe = [r for r in fetch if r["Dispatch_Id"] in ids and "copyBuffer" in r["Kernel_Name"]]
    if not wprobe or not fprobe:
        raise SystemExit("calibration copy not found in the counter runs")
    mean = lambda rs: sum(float(r["Counter_Value"]) for r in rs) / len(rs)  # noqa: E731
    f_scale, w_scale = probe_kib / mean(fprobe), probe_kib / mean(wprobe)
    tag = KERNEL_TAGS.get(kernel, f"{kernel}_kernel<")
    fk, wk = [r for r in fetch if tag in r["Kernel_Name"]], [r for r in write if tag in r["Kernel_Name"]]
    if not fk or not wk:
        raise SystemExit(f"no {kernel} dispatches in the counter runs")
    fetch_kib, write_kib = mean(fk), mean(wk)
    traffic = (fetch_kib * f_scale + write_kib * w_scale) * 1024
    from hyper_connections_amd import traffic as tr
    from hyper_connections_amd import workloads
    wl = workloads.workload(workload)
    per_tok = wl.kind in ("dynamic", "mhc")
    alg = {"pre_mix": tr.pre_bytes(wl.n, wl.d, wl.elem_bytes, per_tok),
           "post_mix": tr.post_bytes(wl.n, wl.d, wl.elem_bytes, per_tok),
           "weights": tr.weights_bytes(wl.n, wl.d, wl.elem_bytes),
           "post_pre_mix": tr.post_pre_bytes(wl.n, wl.d, wl.elem_bytes),
           "post_mix_backward": tr.post_bwd_bytes(wl.n, wl.d, wl.elem_bytes, h_grad=not fold),
           "pre_mix_backward": tr.pre_bwd_bytes(wl.n, wl.d, wl.elem_bytes, True),
           "weights_backward": tr.weights_bwd_bytes(wl.n, wl.d, wl.elem_bytes),
           "weights_backward_stream": tr.weights_bwd_stream_bytes(wl.n, wl.d, wl.elem_bytes)}[kernel] * wl.T
    rec = {"kernel": kernel, "workload": workload, "source_sha": source_sha(kernel),
           "dispatches": {"FETCH_SIZE": len(fk), "WRITE_SIZE": len(wk)},
           "fetch_kib_per_dispatch": round(fetch_kib, 3), "write_kib_per_dispatch": round(write_kib, 3),
           "copy_probe_bytes": COPY_PROBE_BYTES, "fetch_scale": round(f_scale, 5),
           "write_scale": round(w_scale, 5), "traffic_bytes_per_launch": int(round(traffic)),
           "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": round(traffic / alg, 5),
           "commands": cmds}
    base = os.path.join(PROFILES, f"{kernel}_{workload}_counters")
    with open(base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(base + ".md", "w") as fh:
        fh.write(f"# HBM traffic of {kernel}, workload {workload}\n\n")
        fh.write("Commands (run as `cd /tmp && export TMPDIR=/tmp` first; paths are relative to the repository root):\n\n")
        for c in cmds:
            fh.write(f"    {c}\n")
        fh.write(f"\nSummarised with `python bench.py --summarize-counters FETCH_CSV WRITE_CSV "
                 f"--kernel {kernel} --workload {workload}`.\n\n")
        fh.write("| quantity | value |\n|---|---|\n")
        for k in ("fetch_kib_per_dispatch", "write_kib_per_dispatch", "fetch_scale", "write_scale",
                  "traffic_bytes_per_launch", "algorithmic_bytes_per_launch",
                  "traffic_over_algorithmic", "source_sha"):
            fh.write(f"| {k} | {rec[k]} |\n")
        fh.write(f"\nCalibration: the benchmark's {COPY_PROBE_BYTES >> 20} MiB device copy reads "
                 f"FETCH_SIZE x {f_scale:.4f} and WRITE_SIZE x {w_scale:.4f} of its true size; the "
                 "kernel's counters are scaled by the same factors.\n")
    log(f"[bench] wrote {base}.json: traffic {traffic / 1e6:.2f} MB/launch, "
        f"{traffic / alg:.4f} x algorithmic")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="static-bf16")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets (0 = enough to defeat the cache)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle CPU-baseline budget")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--fused", action="store_true",
                    help="fuse each write-back with the next read-mix (chain: every layer; "
                         "static: one step is one fused layer boundary)")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer's gradients: post backward (dF and its records), pre "
                         "backward forming the whole dH, shared-weight sums (static workloads); "
                         "per-token records and the weight producer's gradient as well (dynamic)")
    ap.add_argument("--no-fold", action="store_true",
                    help="with --backward: post backward writes its H gradient and the pre "
                         "backward adds into it (by default post leaves dH to the pre backward, "
                         "which forms the write-back's share from dH' itself)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph (torch.cuda.CUDAGraph) and time replays")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs into profiles/ and exit")
    ap.add_argument("--summarize-mfma", metavar="PMC_CSV",
                    help="summarise a rocprofv3 --pmc run of MFMA/LDS counters into profiles/ and exit")
    ap.add_argument("--kernel", default="post_mix", help="kernel for --summarize-counters/--summarize-mfma")
    ap.add_argument("--command", action="append", default=[],
                    help="profiling command to record in the summary (repeatable)")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.kernel, args.workload, args.command,
                           fold=not args.no_fold)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.kernel, args.workload, args.command)
        return

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this path runs on one GPU "
              "(tokens shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from hyper_connections_amd import hc, traffic, workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    hc.lib()   # raises if the library is not built

    wl = workloads.workload(args.workload)
    n, d, T, s = wl.n, wl.d, wl.T, wl.elem_bytes
    K = wl.K

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        if a.dtype == np.uint8:
            return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
        return torch.from_numpy(a.astype(np.float32)).cuda()

    t0 = time.time()
    inp = workloads.make_inputs(wl)
    log(f"[bench] inputs for {wl.name} generated in {time.time() - t0:.1f}s")
    gamma = dev(inp["gamma"])

    # ---------------------------------------------------------------- sets
    per_tok = wl.kind in ("dynamic", "mhc")
    set_bytes = T * d * s * (2 * n + 2)   # H, F, u, H_out
    sets = args.sets or max(3, math.ceil(2 * MALL_BYTES / set_bytes))
    if wl.kind == "chain":
        sets = 1
    log(f"[bench] {sets} buffer set(s) of {set_bytes / 2 ** 20:.0f} MiB")
    H0 = dev(inp["H"])
    bufs = []
    for i in range(sets):
        b = {"H": H0 if i == 0 else H0.clone(),
             "u": torch.empty((T, d), dtype=H0.dtype, device="cuda"),
             "O": torch.empty_like(H0)}
        if "F" in inp:
            b["F"] = dev(inp["F"]) if i == 0 else bufs[0]["F"].clone()
        else:
            b["F"] = torch.empty((T, d), dtype=H0.dtype, device="cuda")
        if wl.kind == "mhc":
            b["logits"] = dev(inp["logits"]) if i == 0 else bufs[0]["logits"].clone()
        if per_tok:
            b["w"] = torch.empty((T, K), dtype=torch.float32, device="cuda")
        bufs.append(b)
    if wl.kind == "static" or wl.kind == "chain":
        w_static = dev(inp["w"]) if "w" in inp else None
    if wl.kind == "static" and "F" not in inp:
        # the block is tanh of the block input: F computed once, untimed, by
        # the library's own kernels
        F0 = hc.block_tanh(hc.pre_mix(bufs[0]["H"], w_static, gamma, wl.eps))
        for b in bufs:
            b["F"].copy_(F0)
        torch.cuda.synchronize()
    if wl.kind == "dynamic":
        Wp, ws = dev(inp["W"]), dev(inp["w_static"])
    if wl.kind == "chain":
        recs = [dev(workloads.layer_record(wl, l)) for l in range(wl.layers + 1)]

    fold = bool(args.backward) and not args.no_fold
    # algorithmic bytes per launch
    launch_bytes = {
        "pre_mix": traffic.pre_bytes(n, d, s, per_tok) * T,
        "post_mix": traffic.post_bytes(n, d, s, per_tok) * T,
        "post_pre_mix": traffic.post_pre_bytes(n, d, s) * T,
        "weights": traffic.weights_bytes(n, d, s) * T,
        "sinkhorn": traffic.sinkhorn_bytes(n) * T,
        "block_tanh": 2 * d * s * T,
        "post_mix_backward": traffic.post_bwd_bytes(n, d, s, h_grad=not fold) * T,
        "pre_mix_backward": traffic.pre_bwd_bytes(n, d, s, True) * T,
        "weights_backward": traffic.weights_bwd_bytes(n, d, s) * T,
    }

    if args.backward:
        if wl.kind not in ("static", "dynamic") or wl.dtype == "fp8":
            raise SystemExit("--backward is defined for the static and dynamic bf16/fp32 workloads")
        rng = np.random.default_rng(wl.seed + 1)
        G0 = dev(workloads.to_storage(rng.standard_normal((T, n, d), dtype=np.float32), wl.dtype))
        du0 = dev(workloads.to_storage(rng.standard_normal((T, d), dtype=np.float32), wl.dtype))
        ws_bytes = hc.backward_workspace(T, n, d)
        for i, b in enumerate(bufs):
            b["G"] = G0 if i == 0 else G0.clone()
            b["du"] = du0 if i == 0 else du0.clone()
            b["dF"] = torch.empty((T, d), dtype=H0.dtype, device="cuda")
            b["dwp"] = torch.empty(K, dtype=torch.float32, device="cuda")
            b["dwq"] = torch.empty(K, dtype=torch.float32, device="cuda")
            b["dg"] = torch.empty(d, dtype=torch.float32, device="cuda")
            b["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

        if wl.kind == "dynamic":
            # per-token records from a training forward (untimed) that keeps the
            # projections for the backward; gradient records per token
            wws_bytes = int(hc.lib().hc_weights_backward_workspace(T, n, d, 0))
            for b in bufs:
                _, b["saved"] = hc.weights_save(b["H"], Wp, ws, wl.scale, wl.eps, 0, out=b["w"])
                b["dwp"] = torch.empty((T, K), dtype=torch.float32, device="cuda")
                b["dwq"] = torch.empty((T, K), dtype=torch.float32, device="cuda")
                b["dW"] = torch.empty((K, d), dtype=torch.float32, device="cuda")
                b["dws"] = torch.empty(K, dtype=torch.float32, device="cuda")
                b["wws"] = torch.empty(wws_bytes, dtype=torch.uint8, device="cuda")
            torch.cuda.synchronize()
        rec = (lambda b: b["w"]) if wl.kind == "dynamic" else (lambda b: w_static)

        def post_bwd(b):
            # dH lands in b["O"] and the pre backward accumulates into it; folded,
            # the pre backward forms post's share of dH from dH' (b["G"]) itself
            hc.post_mix_backward(b["G"], b["H"], b["F"], rec(b), dH=None if fold else b["O"],
                                 dF=b["dF"], dw=b["dwp"], workspace=b["ws"], h_grad=not fold)

        def pre_bwd(b):
            if fold:
                hc.pre_mix_backward(b["du"], b["H"], rec(b), gamma, wl.eps, dH_out=b["G"],
                                    out=b["O"], dw=b["dwq"], dgamma=b["dg"], workspace=b["ws"])
            else:
                hc.pre_mix_backward(b["du"], b["H"], rec(b), gamma, wl.eps, dH_in=b["O"],
                                    out=b["O"], dw=b["dwq"], dgamma=b["dg"], workspace=b["ws"])

        def weights_bwd(b):
            # the records' gradient from post and pre, through the weight producer
            hc.weights_backward(b["H"], Wp, ws, wl.scale, b["dwp"], wl.eps, 0, dH_in=b["O"],
                                out=b["O"], dW=b["dW"], dw_static=b["dws"], workspace=b["wws"],
                                dw2=b["dwq"], saved=b["saved"])

        ops = [("post_mix_backward", post_bwd), ("pre_mix_backward", pre_bwd)]
        if wl.kind == "dynamic":
            ops.append(("weights_backward", weights_bwd))
    # the kernels of one step, in order: (name, launch on buffer set b)
    elif wl.kind == "static" and args.fused:
        # one layer boundary: write-back of this layer fused with the next read-mix
        ops = [("post_pre_mix", lambda b: hc.post_pre_mix(b["H"], b["F"], w_static, w_static, gamma,
                                                          wl.eps, out=b["O"], u_out=b["u"]))]
    elif wl.kind == "static":
        ops = [("pre_mix", lambda b: hc.pre_mix(b["H"], w_static, gamma, wl.eps, out=b["u"])),
               ("post_mix", lambda b: hc.post_mix(b["H"], b["F"], w_static, out=b["O"]))]
    elif wl.kind == "dynamic":
        ops = [("weights", lambda b: hc.weights(b["H"], Wp, ws, wl.scale, wl.eps, 0, out=b["w"])),
               ("pre_mix", lambda b: hc.pre_mix(b["H"], b["w"], gamma, wl.eps, out=b["u"])),
               ("post_mix", lambda b: hc.post_mix(b["H"], b["F"], b["w"], out=b["O"]))]
    elif wl.kind == "mhc":
        ops = [("sinkhorn", lambda b: hc.sinkhorn(b["logits"], n, wl.iters, out=b["w"])),
               ("pre_mix", lambda b: hc.pre_mix(b["H"], b["w"], gamma, wl.eps, out=b["u"])),
               ("post_mix", lambda b: hc.post_mix(b["H"], b["F"], b["w"], out=b["O"]))]
    else:   # chain: H ping-pongs between b["H"] and b["O"] (an even layer count returns it)
        ops = []
        if args.fused:
            ops.append(("pre_mix", lambda b: hc.pre_mix(b["H"], recs[0], gamma, wl.eps, out=b["u"])))
        for l in range(wl.layers):
            src, dst = ("H", "O") if l % 2 == 0 else ("O", "H")
            ops.append(("block_tanh", lambda b: hc.block_tanh(b["u"], out=b["F"])) if args.fused else
                       ("pre_mix", lambda b, l=l, src=src: hc.pre_mix(b[src], recs[l], gamma, wl.eps,
                                                                       out=b["u"])))
            if args.fused:
                ops.append(("post_pre_mix", lambda b, l=l, src=src, dst=dst: hc.post_pre_mix(
                    b[src], b["F"], recs[l], recs[l + 1], gamma, wl.eps, out=b[dst], u_out=b["u"])))
            else:
                ops.append(("block_tanh", lambda b: hc.block_tanh(b["u"], out=b["F"])))
                ops.append(("post_mix", lambda b, l=l, src=src, dst=dst: hc.post_mix(
                    b[src], b["F"], recs[l], out=b[dst])))

    def step(tm: Timer, i: int):
        b = bufs[i % sets]
        for name, fn in ops:
            tm.run(name, lambda: fn(b))

    # -------------------------------------------------------- copy probe
    cp_n = COPY_PROBE_BYTES
    src = torch.empty(cp_n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * cp_n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    log(f"[bench] device copy (512 MiB read + 512 MiB write): {copy_gbps:.0f} GB/s")

    # ------------------------------------------------------------- timing
    # pass 1: the timed steps, launches back to back (value, ms_per_step)
    # pass 2: the same steps again with events around every launch (per-kernel
    #         durations for the roofline; events add gaps between kernels)
    bare = Timer(torch, per_kernel=False)
    for i in range(args.warmup):
        step(bare, i)
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")
    bare.clear()
    graph = None
    if args.graph:
        # one step captured on torch's capture stream (the binding launches on
        # the current stream); its buffers are fixed, so it always uses set 0
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(bare, 0)
        bare.clear()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
            for name, _ in ops:
                bare.counts[name] = bare.counts.get(name, 0) + 1
        else:
            step(bare, args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    log(f"[bench] {args.steps} timed steps: {ms_step * 1e3:.1f} us/step")

    # pass 2: every kernel of the step on its own, `steps` launches back to
    # back (rotating buffer sets) between one pair of events on the stream
    kms = {}
    for name in dict.fromkeys(k for k, _ in ops):
        fn = next(f for k, f in ops if k == name)
        fn(bufs[0])
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(bufs[i % sets])
        z.record()
        torch.cuda.synchronize()
        kms[name] = a.elapsed_time(z) / args.steps

    hc_kernels = [k for k in kms if k != "block_tanh"]
    launches = {k: c // args.steps for k, c in bare.counts.items()}
    step_bytes = sum(launch_bytes[k] * launches[k] for k in hc_kernels)
    kernels = {}
    for k, ms in kms.items():
        gbps = launch_bytes[k] / (ms * 1e-3) / 1e9
        kernels[k] = {"us": round(ms * 1e3, 2), "launches_per_step": launches[k],
                      "algorithmic_bytes": launch_bytes[k], "gbps": round(gbps, 1),
                      "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        log(f"[bench]   {k:13s} {ms * 1e3:9.2f} us  {gbps:8.0f} GB/s  "
            f"{100 * gbps / HBM_PEAK_GBPS:5.1f}% of 8 TB/s")
    # dominant kernel = largest share of step time
    dom = max(kms, key=lambda k: kms[k] * launches[k])
    dom_gbps = launch_bytes[dom] / (kms[dom] * 1e-3) / 1e9
    # the committed counters of the backward kernels are those of the folded pair
    traffic_b = None if (args.backward and not fold) else counter_traffic(dom, wl.name)

    tokens_per_s = T / (ms_step * 1e-3)
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) inputs, identity-init weights + noise)",
        "config": {"workload": wl.name, "T": T, "n": n, "d": d, "weights": wl.kind,
                   "layers": wl.layers, "buffer_sets": sets, "fused": bool(args.fused),
                   "graph": bool(args.graph), "backward": bool(args.backward),
                   "fold": fold},
        "us_per_layer": round(ms_step * 1e3 / wl.layers, 3),
        "hbm_gbps": round(step_gbps, 1),
        "frac_hbm_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "copy_gbps": round(copy_gbps, 1),
        "gaps_us_per_step": round(ms_step * 1e3 - sum(kms[k] * 1e3 * launches[k] for k in kms), 2),
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_b},
        "cpu_baseline": None,
    }

    # ------------------------------------------------ oracle CPU baseline
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, inp, budget_s: float):
    """The oracle, as it stands, on the host cores: whole passes over the
    workload's tokens (chunks of 1024) until the time budget is used."""
    import numpy as np

    import oracle
    from hyper_connections_amd import workloads

    threads = oracle.get_threads()
    chunk = 1024
    done, t0 = 0, time.perf_counter()
    layers = 0
    while True:
        for c0 in range(0, wl.T, chunk):
            sl = slice(c0, min(wl.T, c0 + chunk))
            H = inp["H"][sl]
            if wl.kind == "static":
                w = inp["w"].astype(np.float64)
                u = oracle.pre_mix(H, w, inp["gamma"], wl.eps)
                if "F" in inp:
                    F = inp["F"][sl]
                else:   # the block is tanh of the block input
                    F = (oracle.round_f32 if wl.dtype == "f32" else oracle.round_bf16)(np.tanh(u))
                oracle.post_mix(H, F, w)
            elif wl.kind == "dynamic":
                w = oracle.weights(H, inp["W"], inp["w_static"].astype(np.float64), wl.scale, wl.eps, 0)
                oracle.pre_mix(H, w, inp["gamma"], wl.eps)
                oracle.post_mix(H, inp["F"][sl], w)
            elif wl.kind == "mhc":
                w = oracle.sinkhorn(inp["logits"][sl].astype(np.float64), wl.n, wl.iters)
                oracle.pre_mix(H, w, inp["gamma"], wl.eps)
                oracle.post_mix(H, inp["F"][sl], w)
            else:
                w = workloads.layer_record(wl, layers % wl.layers).astype(np.float64)
                u = oracle.pre_mix(H, w, inp["gamma"], wl.eps)
                oracle.post_mix(H, oracle.round_bf16(np.tanh(u)), w)
            done += sl.stop - sl.start
            if time.perf_counter() - t0 >= budget_s:
                break
        layers += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    rate = done / el
    if wl.kind == "chain":
        rate /= wl.layers   # one token through all layers
    log(f"[bench] oracle CPU baseline: {done} token passes in {el:.1f}s on {threads} threads")
    return {"value": round(rate, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} token passes of {wl.name} ({wl.T} tokens per full pass, chunks of "
                      f"1024), fp64 oracle, {el:.1f}s wall"}


if __name__ == "__main__":
    main()
