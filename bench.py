#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X (gfx950).

One step = one call of moe_fused_forward (router, permutation, GEMM1 +
SiLU*up, GEMM2, combine) over one batch of synthetic tokens already resident
in HBM.  A default run times the five workloads of the layer's statement one
after another: the Mixtral-shaped prefill batch (M=4096 tokens, K=4096,
N=14336, E=8, top-2, bf16, skewed router) is the headline, and the tiny,
Mixtral-shaped decode, single-token decode and DeepSeek-V3-shaped FP8
batches follow under "workloads" with the same fields.  Per workload: W
untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize(); value = tokens per second.

The same K steps are then replayed from HIP graphs captured from the layer
(graph_ms_per_step, graph_tokens_per_s), the launch mode of a serving loop.
A third pass of K steps through moe_fused_forward_timed records HIP events
between the kernels on the stream they run on; the dominant kernel's mean
duration gives the roofline fraction (algorithmic bytes or FLOPs per launch
/ duration vs the MI355X peak), with the bound taken from the kernel family
the library's plan reports.  The CPU oracle is timed on this host's cores
on a bounded sample of the same workload as a reference point, and the
sample's outputs are checked against it: a run whose output leaves the
tolerance prints "parity_ok": false and exits with status 1.

Prints ONE JSON line.  Only one GPU is used: --gpus N with N > 1 exits.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # dense
STAGES = ["router_logits", "router_topk", "align", "gemm1", "act_quant", "gemm2", "combine"]
METRIC = "fused-MoE layer tokens/s; decode HBM TB/s and prefill MFMA TFLOPS vs peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def hip_runtime():
    import torch
    path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


CPU_SECONDS = 10.0        # oracle work timed for the headline workload's CPU baseline
CPU_SECONDS_EXTRA = 5.0   # and for each of the other workloads of a full run
COPY_BYTES = 1 << 30


def kernel_digest():
    csrc = os.path.join(ROOT, "moe_layer_04_amd", "csrc")
    return source_digest(sorted(os.path.join(csrc, f) for f in os.listdir(csrc)))


def _pmc_rows(path, counter):
    import csv
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"].split("(")[0], []).append(float(r["Counter_Value"]))
    return out


def _request_bytes(path):
    """Bytes the L2 read from memory per dispatch, per kernel, resolved by
    request size: TCC_EA0_RDREQ counts every read request, the _32B / _64B /
    _128B counters the requests of each size (the rest are 64-byte)."""
    import statistics
    c = {n: _pmc_rows(path, n) for n in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum",
                                         "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")}
    out = {}
    for k in c["TCC_EA0_RDREQ_sum"]:
        n = {name: statistics.median(v[k]) for name, v in c.items()}
        n32, n64 = n["TCC_EA0_RDREQ_32B_sum"], n["TCC_EA0_RDREQ_64B_sum"]
        n128 = n["TCC_EA0_RDREQ_128B_sum"]
        rest = n["TCC_EA0_RDREQ_sum"] - n32 - n64 - n128
        out[k] = 32 * n32 + 64 * (n64 + rest) + 128 * n128
    return out


def pmc_summary(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                req_csv=None, copy_req_csv=None):
    """Per-dispatch HBM traffic of the dominant kernel (GEMM1, for one or two
    tokens the GEMM1 that also routes) from counter CSVs.

    Each counter is scaled by what it reads for the plain copy of COPY_BYTES.
    FETCH_SIZE counts a 128-byte read request as 64 bytes on this GPU, so its
    copy factor only holds for kernels whose request mix matches the copy's;
    with the request-size runs (REQ_CSV, COPY_REQ_CSV) the kernel's fetch is
    the request-resolved byte count, checked on the copy against COPY_BYTES."""
    import statistics
    cf = _pmc_rows(copy_fetch_csv, "FETCH_SIZE")
    cw = _pmc_rows(copy_write_csv, "WRITE_SIZE")
    # the copy dispatches are the large ones of the calibration run
    copy_f = max(statistics.median(v) for v in cf.values())
    copy_w = max(statistics.median(v) for v in cw.values())
    f_scale = COPY_BYTES / (copy_f * 1024)
    w_scale = COPY_BYTES / (copy_w * 1024)
    kf = _pmc_rows(fetch_csv, "FETCH_SIZE")
    kw = _pmc_rows(write_csv, "WRITE_SIZE")
    # the dominant kernel: GEMM1 (for one or two tokens the one that also routes)
    name = next(k for k in kf if "gemm1" in k)
    tag = "route_gemm1" if "route_gemm1" in name else "gemm1"
    fetch_counter = statistics.median(kf[name]) * 1024
    fetch = fetch_counter * f_scale
    write = statistics.median(kw[name]) * 1024 * w_scale
    rec = {"kernel": name, "workload": workload, "fetch_size_bytes": fetch_counter,
           "fetch_scale_copy": f_scale, "write_scale": w_scale,
           "dispatches": len(kf[name])}
    if req_csv and copy_req_csv:
        copy_req = max(_request_bytes(copy_req_csv).values())
        rec["copy_request_bytes_over_known"] = copy_req / COPY_BYTES
        fetch = _request_bytes(req_csv)[name]
        rec["fetch_scale_kernel"] = fetch / fetch_counter
    rec.update({"fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
                "bytes_per_launch": fetch + write, "source_digest": kernel_digest()})
    path = os.path.join(ROOT, "profiles", f"{tag}_{workload}_pmc.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def mfma_summary(csv_path, l2_csv=None):
    """MFMA utilisation per kernel from one rocprofv3 --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F8 and
    GRBM_GUI_ACTIVE: the busy cycles (summed over the 1024 SIMDs) over the
    active cycles of one XCD (the aggregated GRBM count covers the 8 XCDs)
    times the SIMDs, the clock those cycles imply over the dispatch, and the
    MFMA FLOPs the hardware executed (512 per MOP, padding rows included);
    with l2_csv (a run of TCC_HIT_sum and TCC_MISS_sum) also the L2 hit rate."""
    import csv
    import statistics
    rows = {}
    for r in csv.DictReader(open(csv_path)):
        k = r["Kernel_Name"].split("(")[0].replace("void ", "")
        d = rows.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    hits = {}
    if l2_csv:
        l2 = {}
        for r in csv.DictReader(open(l2_csv)):
            k = r["Kernel_Name"].split("(")[0].replace("void ", "")
            l2.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = \
                float(r["Counter_Value"])
        for k, disp in l2.items():
            v = [d["TCC_HIT_sum"] / (d["TCC_HIT_sum"] + d["TCC_MISS_sum"]) for d in disp.values()
                 if d.get("TCC_HIT_sum", 0.0) + d.get("TCC_MISS_sum", 0.0) > 0]
            if v:
                hits[k] = statistics.median(v)
    out = []
    for k, disp in rows.items():
        util, clk, flops, rate = [], [], [], []
        for d in disp.values():
            gui = d.get("GRBM_GUI_ACTIVE", 0.0) / 8
            if gui <= 0 or d["ns"] <= 0:
                continue
            util.append(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * 1024))
            clk.append(gui / d["ns"])
            f = 512.0 * (d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) +
                         d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0))
            flops.append(f)
            rate.append(f / d["ns"] / 1e3)
        if not util:
            continue
        rec = {"kernel": k, "dispatches": len(util),
               "mfma_busy_frac": round(statistics.median(util), 4),
               "clock_GHz": round(statistics.median(clk), 3),
               "mfma_flops": statistics.median(flops),
               "mfma_TFLOPs": round(statistics.median(rate), 1)}
        if k in hits:
            rec["l2_hit_rate"] = round(hits[k], 4)
        out.append(rec)
        print(json.dumps(rec))
    return out


def regime_sweep(moe, wlm, wl, dev, ms_list=None):
    """Both kernel families (the workload's bf16, e4m3 or MXFP4 weights) on batches of
    M = 8 .. 1024 tokens (or ms_list) of this workload's shape: mean ms per
    layer call over 10 calls after 3."""
    import torch
    ms_list = ms_list or [8, 16, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024]
    big = wlm.Workload(wl.name + "_sweep", M=max(ms_list), K=wl.K, N=wl.N, E=wl.E,
                       topk=wl.topk, fp8=wl.fp8, fp8_rowwise=wl.fp8_rowwise, mxfp4=wl.mxfp4,
                       seed=wl.seed)
    dtype = (moe.MOE_MXFP4_E2M1 if wl.mxfp4 else moe.MOE_FP8_E4M3_ROWWISE if wl.fp8_rowwise else
             moe.MOE_FP8_E4M3 if wl.fp8 else moe.MOE_BF16)
    g = wlm.generate(big, dev)
    for M in ms_list:
        x = g["x"][:M].contiguous()
        rows = M * wl.topk / wl.E
        row = {"workload": wl.name, "M": M, "rows_per_expert": rows}
        for regime, key in ((moe.MOE_REGIME_DECODE, "decode_ms"),
                            (moe.MOE_REGIME_PREFILL, "tiles_ms")):
            if regime == moe.MOE_REGIME_DECODE and rows > 256:
                continue  # the decode kernels re-stream the weights per 16-row block
            need = moe.workspace_size(dtype, M, wl.K, wl.N, wl.E, wl.topk, regime)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            out = torch.empty((M, wl.K), dtype=torch.bfloat16, device=dev)

            def call():
                moe.moe_fused_forward(x, g["w_router"], None, g["w1"], g["w2"], wl.topk,
                                      w1_scale=g["w1_scale"], w2_scale=g["w2_scale"],
                                      regime=regime, out=out, workspace=ws)

            for _ in range(3):
                call()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(10):
                call()
            torch.cuda.synchronize()
            row[key] = round((time.perf_counter() - t0) * 1e3 / 10, 4)
        print(json.dumps(row), flush=True)


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    help="one workload, or 'all' (default): the Mixtral-shaped prefill batch as "
                         "the headline, then the tiny, Mixtral decode, single-token and "
                         "DeepSeek-shaped FP8 batches under 'workloads'")
    ap.add_argument("--layers", type=int, default=0,
                    help="distinct weight copies stepped round-robin (0 = enough to exceed "
                         "the 256 MB last-level cache several times)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload's shapes with this many tokens M instead")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the oracle's sample (0 = whole batch up to 8)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--fp8", action="store_true",
                    help="the workload with e4m3 weights (one fp32 scale per expert "
                         "tensor) and per-token dynamic e4m3 activations")
    ap.add_argument("--fp8-rowwise", action="store_true",
                    help="with an e4m3 workload: per-channel weight scales (one per output "
                         "row) instead of one per expert tensor")
    ap.add_argument("--mxfp4", action="store_true",
                    help="the workload with MXFP4 weights (e2m1, E8M0 scale per 32 "
                         "elements) and e4m3 activations")
    ap.add_argument("--regime-sweep", action="store_true",
                    help="time the decode and full-tile kernel families (the workload's "
                         "bf16, e4m3 or MXFP4 weights) over batch sizes M = 8 .. 1024 (or "
                         "--sweep-tokens) at this workload's K, N, E, top-k; one JSON line "
                         "per M, then exit")
    ap.add_argument("--sweep-tokens", type=int, nargs="+", default=None,
                    help="batch sizes M of --regime-sweep")
    ap.add_argument("--mfma-summary", nargs="+", metavar="CSV",
                    help="MFMA_CSV [L2_CSV]: MFMA busy fraction, clock and executed MFMA FLOPs "
                         "per kernel from a rocprofv3 --pmc run of SQ_VALU_MFMA_BUSY_CYCLES, "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_INSTS_VALU_MFMA_MOPS_F8 and "
                         "GRBM_GUI_ACTIVE, and the L2 hit rate from a run of TCC_HIT_sum and "
                         "TCC_MISS_sum; one JSON line per kernel, then exit")
    ap.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                    help="FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV [REQ_CSV COPY_REQ_CSV]: "
                         "turn rocprofv3 --pmc counter CSVs of this workload and of the copy "
                         "calibration (FETCH_SIZE, WRITE_SIZE, and optionally the TCC_EA0_RDREQ "
                         "request-size counters) into profiles/gemm1_<workload>_pmc.json and exit")
    args = ap.parse_args()
    if args.mfma_summary:
        if len(args.mfma_summary) > 2:
            sys.exit("--mfma-summary takes MFMA_CSV [L2_CSV]")
        mfma_summary(*args.mfma_summary)
        return
    if args.pmc_summary:
        if len(args.pmc_summary) not in (4, 6):
            ap.error("--pmc-summary takes 4 or 6 CSV paths")
        if args.workload == "all":
            ap.error("--pmc-summary takes one --workload")
        pmc_summary(args.workload, *args.pmc_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import moe_layer_04_amd as moe
    from moe_layer_04_amd import workloads as wlm

    if args.workload != "all" and args.workload not in wlm.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; 'all' or one of {list(wlm.WORKLOADS)}")
    if args.workload == "all" and (args.fp8 or args.fp8_rowwise or args.mxfp4 or args.tokens or
                                   args.regime_sweep or args.pmc_summary):
        sys.exit("--fp8, --fp8-rowwise, --mxfp4, --tokens, --regime-sweep and --pmc-summary "
                 "take one --workload")
    wl = wlm.WORKLOADS["mixtral_prefill" if args.workload == "all" else args.workload]
    if args.fp8 and not wl.fp8:
        wl = wl.resized(name=wl.name + "_fp8", fp8=True)
    if args.fp8_rowwise:
        if not wl.fp8:
            sys.exit("--fp8-rowwise needs an e4m3 workload")
        wl = wl.resized(name=wl.name + "_rowwise", fp8_rowwise=True)
    if args.mxfp4:
        wl = wl.resized(name=wl.name + "_mxfp4", fp8=False, fp8_rowwise=False, mxfp4=True)
    if args.tokens:
        wl = wl.resized(name=f"{wl.name}_M{args.tokens}", M=args.tokens)
    if not torch.cuda.is_available():
        sys.exit("no GPU visible")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "reps": 3}))
        return
    moe.load_library(build_if_missing=True)
    if args.regime_sweep:
        regime_sweep(moe, wlm, wl, dev, args.sweep_tokens)
        return

    hip = hip_runtime()
    if args.workload == "all":
        names = ["mixtral_prefill"] + [n for n in wlm.WORKLOADS if n != "mixtral_prefill"]
        wls = [wlm.WORKLOADS[n] for n in names]
    else:
        wls = [wl]
    records = []
    for i, w in enumerate(wls):
        cpu_s = 0.0 if args.no_cpu_baseline else (CPU_SECONDS if i == 0 else CPU_SECONDS_EXTRA)
        records.append(bench_workload(moe, wlm, w, args, dev, hip, cpu_s))
        torch.cuda.empty_cache()
    result = dict(records[0])
    if len(records) > 1:
        # the headline is the first (the prefill batch, the matrix-core half of
        # the metric); the other workloads of the same run follow with the
        # same fields
        result["workloads"] = {r["config"]["workload"]: {k: v for k, v in r.items()
                                                          if k not in HEADLINE_ONLY}
                               for r in records[1:]}
    bad = [r["config"]["workload"] for r in records
           if r.get("parity_vs_oracle") and not r["parity_vs_oracle"]["ok"]]
    result["parity_ok"] = not bad
    print(json.dumps(result), flush=True)
    if bad:
        log(f"output outside the oracle tolerance on {bad}")
        sys.exit(1)


HEADLINE_ONLY = ("metric", "unit", "n_gpus", "steps", "warmup", "higher_is_better", "scaling",
                 "vs_baseline", "data")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_workload(moe, wlm, wl, args, dev, hip, cpu_seconds):
    """One workload: K timed steps after W warm-up steps, the same steps from
    captured HIP graphs, a pass with HIP events between the kernels, and the
    oracle on a bounded sample.  Returns the workload's record."""
    import numpy as np
    import torch

    log(f"generating {wl}")
    g = wlm.generate(wl, dev)
    wbytes = 0.5 + 1 / 32 if wl.mxfp4 else (1 if wl.fp8 else 2)   # weight + block-scale bytes
    dtype_name = "mxfp4/e4m3" if wl.mxfp4 else ("fp8" if wl.fp8 else "bf16")
    dtype = (moe.MOE_MXFP4_E2M1 if wl.mxfp4 else
             moe.MOE_FP8_E4M3_ROWWISE if wl.fp8_rowwise else
             moe.MOE_FP8_E4M3 if wl.fp8 else moe.MOE_BF16)
    plan = moe.fused_plan(dtype, wl.M, wl.K, wl.N, wl.E, wl.topk)

    # routing of this batch (for the realised active-expert count)
    ids, _, _ = moe.moe_topk(g["x"], g["w_router"], g["bias"], wl.topk)
    torch.cuda.synchronize()
    active = int(torch.unique(ids).numel())
    w1_e = int(2 * wl.N * wl.K * wbytes)
    w2_e = int(wl.K * wl.N * wbytes)
    touched = active * (w1_e + w2_e)
    layers = args.layers or max(1, min(8, math.ceil(2 * 2**30 / touched)))
    w1s = [g["w1"]] + [g["w1"].clone() for _ in range(layers - 1)]
    w2s = [g["w2"]] + [g["w2"].clone() for _ in range(layers - 1)]
    log(f"active experts {active}, {touched / 1e9:.3f} GB of weights per step, {layers} layer(s)")

    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((wl.M, wl.K), dtype=torch.bfloat16, device=dev)

    def step(i):
        moe.moe_fused_forward(g["x"], g["w_router"], g["bias"], w1s[i % layers], w2s[i % layers],
                              wl.topk, w1_scale=g["w1_scale"], w2_scale=g["w2_scale"], out=out,
                              workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = wl.M * args.steps / elapsed
    log(f"{wl.name}: {ms_per_step:.4f} ms per step")

    # ---- the same steps replayed from captured HIP graphs (one per weight copy)
    graphs = [moe.FusedForwardGraph(g["x"], g["w_router"], g["bias"], w1s[L], w2s[L], wl.topk,
                                    w1_scale=g["w1_scale"], w2_scale=g["w2_scale"])
              for L in range(layers)]
    for i in range(args.warmup):
        graphs[i % layers].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % layers].replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del graphs

    # ---- per-kernel durations from HIP events on the layer's stream --------
    lib = moe.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    nev = len(STAGES) + 1
    evs = []
    for _ in range(args.steps):
        arr = (ctypes.c_void_p * nev)()
        for j in range(nev):
            h = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(h)) == 0
            arr[j] = h
        evs.append(arr)
    nbytes = ctypes.c_size_t(ws.numel())

    def P(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    torch.cuda.synchronize()
    for i in range(args.steps):
        L = i % layers
        rc = lib.moe_fused_forward_timed(P(g["x"]), P(g["w_router"]), P(g["bias"]), P(w1s[L]),
                                         P(w2s[L]), P(g["w1_scale"]), P(g["w2_scale"]), dtype,
                                         wl.M, wl.K, wl.N, wl.E, wl.topk, 0, P(out), P(ws),
                                         ctypes.byref(nbytes), stream, evs[i])
        assert rc == 0, moe.status_string(rc)
    torch.cuda.synchronize()
    stage_ms = {s: [] for s in STAGES}
    total_ms = []
    for arr in evs:
        f = ctypes.c_float()
        for j, s in enumerate(STAGES):
            assert hip.hipEventElapsedTime(ctypes.byref(f), arr[j], arr[j + 1]) == 0
            stage_ms[s].append(f.value)
        assert hip.hipEventElapsedTime(ctypes.byref(f), arr[0], arr[nev - 1]) == 0
        total_ms.append(f.value)
        for j in range(nev):
            hip.hipEventDestroy(arr[j])
    kern_us = {s: float(np.mean(v)) * 1e3 for s, v in stage_ms.items()}
    if plan.fused_decode:
        # three launches: router + top-k + align + GEMM1 in one kernel
        # (recorded as the first stage; stages 2-5 are empty), GEMM2, combine
        kern_us = {"route_gemm1": kern_us["router_logits"], "gemm2": kern_us["gemm2"],
                   "combine": kern_us["combine"]}

    # ---- algorithmic work and roofline --------------------------------------
    slots = wl.M * wl.topk
    alg_bytes = (touched + wl.M * wl.K * 2 * 2 + wl.E * wl.K * 2
                 + (wl.E * 4 if wl.bias_var else 0)
                 + ((wl.E * (2 * wl.N + wl.K) * 4 if wl.fp8_rowwise else 2 * wl.E * 4)
                    if wl.fp8 else 0))
    alg_flops = 6.0 * slots * wl.N * wl.K
    step_s = ms_per_step / 1e3
    # the bound of the dominant kernel follows the kernel family the library
    # ran (its plan): the Swap-AB decode kernels stream weights, the full
    # tiles are matrix-core bound
    decode = plan.regime == moe.MOE_REGIME_DECODE
    mfma_peak = MFMA_PEAK_TFLOPS["bf16" if dtype_name == "bf16" else "fp8"]
    if decode:
        g1_s = kern_us["route_gemm1" if plan.fused_decode else "gemm1"] / 1e6
        # GEMM1 reads W1 of every active expert once plus the token rows
        g1_bytes = active * w1_e + wl.M * wl.K * (1 if (wl.fp8 or wl.mxfp4) else 2)
        achieved = g1_bytes / g1_s / 1e9
        roofline = {"bound": "hbm", "kernel": "route_gemm1" if plan.fused_decode else "gemm1",
                    "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "units_per_launch": active, "bytes_per_unit": w1_e}
    else:
        g1_s = kern_us["gemm1"] / 1e6
        g1_flops = 4.0 * slots * wl.N * wl.K
        achieved = g1_flops / g1_s / 1e12
        roofline = {"bound": "mfma", "kernel": "gemm1", "achieved": round(achieved, 1),
                    "peak": mfma_peak, "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4),
                    "traffic": None, "units_per_launch": slots,
                    "flops_per_unit": 4.0 * wl.N * wl.K}
    # HBM traffic from committed counter runs, only while the kernels are unchanged
    digest = kernel_digest()
    pmc = os.path.join(ROOT, "profiles", f"{roofline['kernel']}_{wl.name}_pmc.json")
    if os.path.exists(pmc):
        rec = json.load(open(pmc))
        if rec.get("source_digest") == digest:
            roofline["traffic"] = rec.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic (seeded N(0,1/fan_in) weights, random init; no dataset)",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "E": wl.E,
                   "topk": wl.topk, "weights": ("mxfp4 (e2m1, E8M0 per 32)" if wl.mxfp4 else
                               ("e4m3 per-channel" if wl.fp8_rowwise else "e4m3 per-tensor")
                               if wl.fp8 else "bf16"),
                   "router_bias_var": wl.bias_var, "seed": wl.seed, "layers": layers,
                   "active_experts": active},
        "kernel_family": ("swap-ab decode, routing inside GEMM1" if plan.fused_decode else
                          "swap-ab decode" if decode else "full tiles"),
        "block_m": plan.block_m,
        # both fractions of the whole step: algorithmic bytes over the step
        # time against 8 TB/s, algorithmic FLOPs against the dense MFMA peak
        "step_hbm_GBps": round(alg_bytes / step_s / 1e9, 1),
        "step_hbm_frac": round(alg_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_tflops": round(alg_flops / step_s / 1e12, 2),
        "step_mfma_frac": round(alg_flops / step_s / 1e12 / mfma_peak, 4),
        "algorithmic_bytes": alg_bytes,
        "algorithmic_flops": alg_flops,
        "kernel_us": {k: round(v, 2) for k, v in kern_us.items()},
        "timed_pass_ms_per_step": round(float(np.mean(total_ms)), 4),
        # per-call spread of the same pass: HIP events before the first and
        # after the last kernel of each call (back to back, weights cycled
        # over the layer copies)
        "call_ms": {q: round(float(np.percentile(total_ms, v)), 4)
                    for q, v in (("p10", 10), ("p50", 50), ("p90", 90))},
        "graph_ms_per_step": round(graph_ms, 4),
        "graph_tokens_per_s": round(wl.M / (graph_ms / 1e3), 1),
        "roofline": roofline,
        "source_digest": digest,
    }

    # ---- CPU oracle on a bounded sample -------------------------------------
    if cpu_seconds > 0:
        import oracle
        n_tok = args.cpu_tokens or min(wl.M, 8)
        toks = list(range(n_tok))
        x_h = wlm.to_numpy_bits(g["x"])
        wr_h = wlm.to_numpy_bits(g["w_router"])
        bias_h = None if g["bias"] is None else g["bias"].cpu().numpy()
        rids, _ = oracle.topk(oracle.logits(x_h[toks], wr_h, bias_h), wl.topk)
        need_e = sorted(set(rids.reshape(-1).tolist()))
        w1h = [wlm.to_numpy_bits(g["w1"][e]) if e in need_e else None for e in range(wl.E)]
        w2h = [wlm.to_numpy_bits(g["w2"][e]) if e in need_e else None for e in range(wl.E)]
        s1 = None if g["w1_scale"] is None else g["w1_scale"].cpu().numpy()
        s2 = None if g["w2_scale"] is None else g["w2_scale"].cpu().numpy()
        log(f"oracle on {n_tok} token(s), {len(need_e)} expert(s)")
        # the sample is evaluated repeatedly until about cpu_seconds of work
        reps = 0
        t0 = time.perf_counter()
        while True:
            ref, _, _ = oracle.moe_forward(x_h, wr_h, bias_h, w1h, w2h, wl.topk, w1_scale=s1,
                                           w2_scale=s2, tokens=toks, fp8=wl.fp8,
                                           mxfp4=wl.mxfp4)
            reps += 1
            if time.perf_counter() - t0 >= cpu_seconds:
                break
        cpu_s = time.perf_counter() - t0
        got = out.float().cpu().numpy()[toks].astype(np.float64)
        den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
        err = float((np.abs(got - ref).max(axis=1) / den).max())
        tol = 6e-2 if (wl.fp8 or wl.mxfp4) else 2e-2
        result["cpu_baseline"] = {
            "value": round(n_tok * reps / cpu_s, 3), "unit": "tokens/s",
            "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"first {n_tok} of the {wl.M} tokens of the same batch "
                      f"({n_tok * wl.topk} token-slots, fp64), evaluated {reps} times",
            "seconds": round(cpu_s, 3)}
        result["parity_vs_oracle"] = {"max_row_rel_err": err, "tokens": n_tok, "tol": tol,
                                      "ok": bool(np.isfinite(got).all() and err <= tol)}
    # the padded row count of this batch's routing, from the workspace (the
    # number of token blocks the GEMMs ran over)
    npad = int(moe.fused_routing(ws, plan, wl.M, wl.E, wl.topk)["num_padded"].item())
    result["routed_blocks"] = npad // plan.block_m
    del g, w1s, w2s, ws, out
    return result


if __name__ == "__main__":
    main()
