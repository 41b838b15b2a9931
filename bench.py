#!/usr/bin/env python3
"""Benchmark of the BF16 x NVFP4 GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 50]

A step is one decode pass of the GEMM hot path over the four linear layers of
a Llama-3-70B block at m = 16 (fused QKV 10240x8192, O 8192x8192, fused
gate/up 57344x8192, down 8192x28672; NVFP4 weights, synthetic seeded inputs of
the Petit blog's GEMM workload, section "Detailed performance analysis").
Protocol from the same section: 50 warm-up runs, mean over 100 timed runs.
Every launch reads a different copy of its layer's packed weights (copies per
layer >= 1 GiB in total) so the 256 MB last-level cache cannot serve them.

Printed as the last stdout line, one JSON object:
  value        aggregate algorithmic HBM GB/s of the decode step
               (bytes = N*K/2 codes + N*K/16 scales + 2*m*K + 2*m*N per GEMM)
  roofline     the gate/up GEMM (largest share of the step): algorithmic bytes
               per launch / mean launch time, from HIP events on the launch
               stream around a run of back-to-back gate/up launches that
               follows the timed steps, against 8 TB/s; traffic = HBM bytes
               per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters kept
               in profiles/, reported only while the kernel sources still
               hash to the value they were measured on
  prefill      the same four layers at m = 256: TFLOP/s against the 2.5
               PFLOP/s dense BF16 matrix-core peak
  fp16         the same decode step and prefill with FP16 activations and
               output (fp4_gemm_f16; FP16 matrix-core peak 2.5 PFLOP/s)
  quantize     the offline quantizer (fp4_quantize) on the gate/up weight
               (57344 x 8192 BF16): GB/s of BF16 read + codes and scales
               written, both formats
  native       (with --native) the native FP4 path (fp4_gemm_native: activations quantized
               to MXFP4, FP4 x FP4 matrix cores, MXFP4 weights) on the same
               four layer shapes at m = 256 (TFLOP/s against the 10.1
               PFLOP/s dense FP4 peak) and m = 16 (GB/s)
  moe          the grouped MoE GEMM (fp4_moe_gemm): 128 experts, top-4,
               fused gate/up N = 5760, K = 2880, MXFP4, 16 and 256 tokens;
               algorithmic bytes = the routed-to experts' packed weights +
               gathered activations + outputs
  cpu_baseline the CPU oracle (float64 NumPy) timed on a bounded sample
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 matrix-core peak
METRIC = "BF16×NVFP4 GEMM: HBM GB/s at m=16, TFLOP/s at m=256, % of roofline"
ROTATE_BYTES = 1 << 30


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_gemm_decode_gate_up_nvfp4_m16.json")


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter record, or None
    when the kernel sources changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        return rec["hbm_bytes_per_launch"] if sources_sha256(rec["sources"]) == rec["source_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


KERNEL_SOURCES = ["mixed_precision_bf16_amd/csrc/kernels.h", "mixed_precision_bf16_amd/csrc/layout.h",
                  "mixed_precision_bf16_amd/csrc/dispatch.h", "mixed_precision_bf16_amd/csrc/decode_inst.inc",
                  "mixed_precision_bf16_amd/csrc/decode_bf16.hip", "mixed_precision_bf16_amd/csrc/prefill_inst.inc",
                  "mixed_precision_bf16_amd/csrc/prefill_bf16.hip", "mixed_precision_bf16_amd/csrc/fp4gemm.hip"]
COUNTER_RECORD = os.path.join(ROOT, "profiles", "counters_gemm_prefill_decode_nvfp4.json")
GATE_UP_DECODE_KERNEL = "gemm_decode<0, 0, 1, 2, 7, 2, false>"


def sources_sha256(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def _counter_rows(d):
    import csv
    import glob
    (path,) = glob.glob(os.path.join(d, "*_counter_collection.csv"))
    return list(csv.DictReader(open(path)))


def traffic_record(fetch_dir, write_dir):
    """FETCH_SIZE and WRITE_SIZE passes (rocprofv3 --pmc, one counter per run,
    each run starting with the 256 MiB calibration copy of --calibrate-copy)
    -> the HBM bytes per gate/up decode launch, each counter scaled by what it
    reads for the copy of known size; written to TRAFFIC_RECORD with the
    SHA-256 of the kernel sources."""
    import statistics
    out = {}
    for d, name in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == name]
        copy = [float(r["Counter_Value"]) for r in rows if "__amd_rocclr_copyBuffer" in r["Kernel_Name"]]
        gu = [float(r["Counter_Value"]) for r in rows if GATE_UP_DECODE_KERNEL in r["Kernel_Name"]]
        out[name] = (copy[0], statistics.mean(gu), len(gu))
    cb = 256 << 20
    ff, wf = cb / (out["FETCH_SIZE"][0] * 1024), cb / (out["WRITE_SIZE"][0] * 1024)
    hbm = int(round(out["FETCH_SIZE"][1] * 1024 * ff + out["WRITE_SIZE"][1] * 1024 * wf))
    rec = {"kernel": "gemm_decode<0,0,1,2,7,2> (gate_up 57344x8192, m=16, NVFP4, BF16 activations)",
           "sources": KERNEL_SOURCES, "source_sha256": sources_sha256(KERNEL_SOURCES),
           "command": "cd /tmp && rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <fetch> -o f -- "
                      "python3 <repo>/bench.py --calibrate-copy --steps 3 --warmup 1 --no-prefill --no-cpu-baseline "
                      "--no-fp16 --no-moe --no-quantize --no-blas --no-configs  (then the same with --pmc WRITE_SIZE "
                      "into <write>); python3 bench.py --traffic-record <fetch> <write>",
           "calibration": {"copy_bytes": cb, "copy_fetch_kib": out["FETCH_SIZE"][0],
                           "copy_write_kib": out["WRITE_SIZE"][0], "fetch_factor": round(ff, 6),
                           "write_factor": round(wf, 6)},
           "fetch_kib_per_dispatch_mean": round(out["FETCH_SIZE"][1], 2),
           "write_kib_per_dispatch_mean": round(out["WRITE_SIZE"][1], 2),
           "dispatches": out["FETCH_SIZE"][2], "hbm_bytes_per_launch": hbm,
           "algorithmic_bytes_per_launch": algorithmic_bytes(16, 57344, 8192, 16)}
    json.dump(rec, open(TRAFFIC_RECORD, "w"), indent=1)
    open(TRAFFIC_RECORD, "a").write("\n")
    return rec


def counter_record(pmc_dir):
    """One SQ counter pass (rocprofv3 --pmc ... --kernel-trace) -> per kernel
    instantiation and grid (one row per layer) the means per dispatch of every
    counter and of the duration; written to COUNTER_RECORD with the SHA-256 of
    the kernel sources."""
    import csv
    import glob
    import statistics
    rows = _counter_rows(pmc_dir)
    (tpath,) = glob.glob(os.path.join(pmc_dir, "*_kernel_trace.csv"))
    dur = {r["Dispatch_Id"]: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
           for r in csv.DictReader(open(tpath))}
    per = {}  # dispatch -> (kernel, grid, {counter: value})
    for r in rows:
        if "fp4::" not in r["Kernel_Name"]:
            continue
        name = r["Kernel_Name"].split("(")[0].replace("void fp4::", "")
        d = per.setdefault(r["Dispatch_Id"], (name, int(r["Grid_Size"]), {}))
        d[2][r["Counter_Name"]] = float(r["Counter_Value"])
    groups = {}  # one row per layer: kernel, grid and matrix-instruction count identify it
    for i, (name, grid, cnt) in per.items():
        groups.setdefault((name, grid, int(cnt.get("SQ_INSTS_MFMA", 0))), []).append(i)
    table = []
    for (name, grid, mfma), ids in sorted(groups.items()):
        ent = {"kernel": name, "grid_threads": grid, "dispatches": len(ids),
               "us_mean": round(statistics.mean(dur[i] for i in ids if i in dur), 2)}
        for c in per[ids[0]][2]:
            ent[c] = statistics.mean(per[i][2][c] for i in ids)
        table.append(ent)
    rec = {"sources": KERNEL_SOURCES, "source_sha256": sources_sha256(KERNEL_SOURCES),
           "command": "cd /tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU "
                      "SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --kernel-trace "
                      "--output-format csv -d <pmc> -o p -- python3 <repo>/bench.py --steps 3 --warmup 1 "
                      "--no-cpu-baseline --no-fp16 --no-moe --no-quantize --no-blas --no-configs "
                      "--prefill-launches 3; python3 bench.py --counter-record <pmc>",
           "kernels": table}
    json.dump(rec, open(COUNTER_RECORD, "w"), indent=1)
    open(COUNTER_RECORD, "a").write("\n")
    return rec


def algorithmic_bytes(m, N, K, G):
    return N * K // 2 + N * K // G + 2 * m * K + 2 * m * N


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--prefill-launches", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16", action="store_true", help="skip the FP16-activation decode and prefill lines")
    ap.add_argument("--no-moe", action="store_true", help="skip the grouped MoE GEMM lines")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the MXFP4 decode sweep and the ragged-shape roofline fractions")
    ap.add_argument("--no-blas", action="store_true",
                    help="skip the BF16 hipBLASLt comparison and the measured copy / GEMM ceilings")
    ap.add_argument("--no-quantize", action="store_true", help="skip the quantizer line")
    ap.add_argument("--native", action="store_true", help="also time the native FP4 path (opt-in)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first (known bytes for HBM counter scaling)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the gate/up traffic record from two rocprofv3 counter passes, then exit (no GPU)")
    ap.add_argument("--counter-record", metavar="PMC_DIR",
                    help="write the SQ counter record from a rocprofv3 counter pass, then exit (no GPU)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Layer:
    """Packed weights of one layer, rotated over R device copies."""

    def __init__(self, prob, F, torch):
        self.name, self.N, self.K, self.fmt, self.G = prob.name.split("_m")[0], prob.N, prob.K, prob.fmt, prob.group
        wq, sq = F.repack(prob.codes, prob.scales, prob.N, prob.K, prob.fmt)
        wq_d, sq_d = F.upload(wq, sq)
        self.R = max(1, math.ceil(ROTATE_BYTES / (wq.size + sq.size)))
        self.wq = [wq_d] + [wq_d.clone() for _ in range(self.R - 1)]
        self.sq = [sq_d] + [sq_d.clone() for _ in range(self.R - 1)]


def make_call(F, torch, layer, A, C, r, ws, entry="fp4_gemm"):
    """Pre-marshalled fp4_gemm (or fp4_gemm_f16) call on torch's current stream."""
    lib = F.lib()
    stream = F._c_vp(torch.cuda.current_stream().cuda_stream)
    m = A.shape[0]
    ws_bytes = ws.numel() if ws is not None else 0
    args = (F._dev_ptr(A), F._dev_ptr(layer.wq[r]), F._dev_ptr(layer.sq[r]), F._dev_ptr(C), m, layer.N, layer.K,
            layer.fmt, F._dev_ptr(ws), ws_bytes, stream)
    fn = getattr(lib, entry)

    def call():
        st = fn(*args)
        if st:
            F._check(st, entry)
    return call


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(decode_layers_probs):
    """The oracle as it stands (float64 NumPy: dequant + library matmul) on a
    bounded sample: m = 16 against the first 8192 rows of the gate/up weights,
    on all host cores available to the process (BLAS threads set to match)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    blas = {"vendor": "unknown", "threads": None}
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = {"vendor": info[0].get("internal_api", "unknown"),
                    "threads": max(p.get("num_threads", 1) for p in info)}
    except Exception:  # noqa: BLE001
        pass
    p = decode_layers_probs[2]
    rows = 8192
    codes, scales = p.codes[:rows], p.scales[:rows]
    reps, times = 0, []
    t_start = time.perf_counter()
    try:
        while reps < 3 or (time.perf_counter() - t_start < 10.0 and reps < 30):
            t0 = time.perf_counter()
            oracle.gemm_reference(p.a_bits, codes, scales, p.K, p.fmt)
            times.append(time.perf_counter() - t0)
            reps += 1
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    t = float(np.mean(times))
    b = algorithmic_bytes(p.m, rows, p.K, p.group)
    return {"value": round(b / t / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "blas_vendor": blas["vendor"], "blas_threads": blas["threads"],
            "sample": f"m=16 x first {rows} rows of the gate_up weights (K={p.K}), float64 NumPy dequant + "
                      f"matmul, mean of {reps} runs ({t:.2f} s each); the elementwise dequant runs on one "
                      f"thread, the matmul on {blas['threads']} {blas['vendor']} threads "
                      f"({cores} cores in the process's affinity set)",
            "seconds_per_run": round(t, 3)}


def timed(calls_fn, n):
    """Mean microseconds per call of n back-to-back calls (HIP events on the
    current stream)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(n):
        calls_fn(s)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def fp16_lines(args, F, torch, layers, A_bf16, WS, dev, m):
    """Decode step (m = 16) and prefill (m = 256) with FP16 activations: the
    BF16 activations converted to FP16, the same packed weights, rotation and
    protocol as the BF16 lines."""
    A = [a.to(torch.float16) for a in A_bf16]
    C = [torch.empty((m, l.N), dtype=torch.float16, device=dev) for l in layers]
    calls = [[make_call(F, torch, l, A[i], C[i], r, WS[i], "fp4_gemm_f16") for r in range(l.R)]
             for i, l in enumerate(layers)]

    def step(s):
        for i, l in enumerate(layers):
            calls[i][s % l.R]()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    us_step = timed(step, args.steps)
    bytes_step = sum(algorithmic_bytes(m, l.N, l.K, l.G) for l in layers)
    gbs = bytes_step / (us_step * 1e-6) / 1e9
    out = {"decode_step_us": round(us_step, 2), "decode_GB/s": round(gbs, 1),
           "decode_frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    if not args.no_prefill:
        mp = 256
        rng = np.random.Generator(np.random.PCG64(2_000_000))
        tot_f, tot_t = 0.0, 0.0
        for l in layers:
            a = torch.from_numpy(rng.standard_normal((mp, l.K), dtype=np.float32)).to(torch.float16).to(dev)
            c = torch.empty((mp, l.N), dtype=torch.float16, device=dev)
            ws = F.new_workspace(mp, l.N, l.K, l.fmt, device=dev)
            pc = [make_call(F, torch, l, a, c, r, ws, "fp4_gemm_f16") for r in range(l.R)]
            for s in range(5):
                pc[s % l.R]()
            tot_t += timed(lambda s: pc[s % l.R](), args.prefill_launches)
            tot_f += 2.0 * mp * l.N * l.K
        out["prefill_TFLOP/s"] = round(tot_f / tot_t / 1e6, 1)
        out["prefill_frac_mfma"] = round(tot_f / tot_t / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)
    return out


def quantize_lines(args, F, torch, dev):
    """fp4_quantize on a 57344 x 8192 BF16 weight drawn N(0, 1) on the device;
    mean of back-to-back launches alternating two weight copies (2 x 940 MB,
    beyond the last-level cache).  Algorithmic bytes: 2 per weight read, 1/2
    per weight of codes and 1/G of scales written."""
    N, K = 57344, 8192
    gen = torch.Generator(device=dev)
    gen.manual_seed(99)
    Ws = [torch.randn((N, K), device=dev, generator=gen).to(torch.bfloat16) for _ in range(2)]
    lib = F.lib()
    stream = F._c_vp(torch.cuda.current_stream().cuda_stream)
    out = {"N": N, "K": K}
    for fmt, G in ((0, 16), (1, 32)):
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((N, K // G), dtype=torch.uint8, device=dev)
        argv = [(F._dev_ptr(W), F._dev_ptr(codes), F._dev_ptr(scales), N, K, fmt, 1.0, stream) for W in Ws]

        def call(s, argv=argv):
            st = lib.fp4_quantize(*argv[s % 2])
            if st:
                F._check(st, "fp4_quantize")
        for s in range(3):
            call(s)
        torch.cuda.synchronize()
        us = timed(call, args.prefill_launches)
        b = N * K * 2 + N * K // 2 + N * K // G
        out["nvfp4" if fmt == 0 else "mxfp4"] = {"us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                                                 "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
    del Ws
    torch.cuda.empty_cache()
    return out


MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix-core peak


def native_lines(args, F, torch, dev):
    """fp4_gemm_native on the four Llama-3-70B layer shapes with MXFP4 weights
    made as random packed bytes on the device (E8M0 bytes 121 .. 129; the
    timing does not depend on the values, the GPU tests cover these shapes
    with seeded inputs), rotating copies of >= 1 GiB per layer; activations
    N(0, 1) in BF16, quantized inside every call."""
    shapes = (("qkv", 10240, 8192), ("o", 8192, 8192), ("gate_up", 57344, 8192), ("down", 8192, 28672))
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    lib = F.lib()
    stream = F._c_vp(torch.cuda.current_stream().cuda_stream)
    out = {"weights": "mxfp4 (native layout)", "activations": "bf16, quantized to mxfp4 per call",
           "peak_TFLOP/s": MFMA_FP4_PEAK_TFLOPS, "layers": {}}
    tot = {16: [0.0, 0.0], 256: [0.0, 0.0]}
    for name, N, K in shapes:
        nw, ns = F.repack_size(N, K, 1)
        R = max(1, math.ceil(ROTATE_BYTES / (nw + ns)))
        copies = [(torch.randint(0, 256, (nw,), dtype=torch.uint8, device=dev, generator=gen),
                   torch.randint(121, 130, (ns,), dtype=torch.uint8, device=dev, generator=gen)) for _ in range(R)]
        rec = {}
        for m in (16, 256):
            a = torch.randn((m, K), device=dev, generator=gen).to(torch.bfloat16)
            c = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            wsb = F.native_workspace_size(m, N, K)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
            argv = [(F._dev_ptr(a), F._dev_ptr(wq), F._dev_ptr(sq), F._dev_ptr(c), m, N, K, 1.0, F._dev_ptr(ws), wsb,
                     stream) for wq, sq in copies]

            def call(s_, argv=argv):
                st = lib.fp4_gemm_native(*argv[s_ % len(argv)])
                if st:
                    F._check(st, "fp4_gemm_native")
            for s_ in range(3):
                call(s_)
            torch.cuda.synchronize()
            us = timed(call, args.prefill_launches)
            fl = 2.0 * m * N * K
            b = algorithmic_bytes(m, N, K, 32)
            rec[f"m{m}"] = {"us": round(us, 2), "TFLOP/s": round(fl / us / 1e6, 1),
                            "frac_fp4_mfma": round(fl / us / 1e6 / MFMA_FP4_PEAK_TFLOPS, 4),
                            "GB/s": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
            tot[m][0] += fl if m == 256 else b
            tot[m][1] += us
        out["layers"][name] = rec
        del copies
        torch.cuda.empty_cache()
    out["prefill_TFLOP/s"] = round(tot[256][0] / tot[256][1] / 1e6, 1)
    out["prefill_frac_fp4_mfma"] = round(tot[256][0] / tot[256][1] / 1e6 / MFMA_FP4_PEAK_TFLOPS, 4)
    out["decode_GB/s"] = round(tot[16][0] / tot[16][1] / 1e3, 1)
    out["decode_frac_hbm"] = round(tot[16][0] / tot[16][1] / 1e3 / HBM_PEAK_GBS, 4)
    return out


def blas_lines(args, torch, layers, per_layer, prefill, dev):
    """Context for the Petit blog's own comparison ("Detailed performance
    analysis": the FP4 kernel against the vendor BF16 GEMM at m = 16 and 256):
    torch.matmul with BF16 weights of the same shapes (hipBLASLt on ROCm) on
    this GPU, same rotation of weight copies, and the speed-up of fp4_gemm."""
    gen = torch.Generator(device=dev).manual_seed(3)
    out = {"library": "torch.matmul bf16 x bf16 (hipBLASLt)", "layers": {}}
    for l in layers:
        R = max(2, math.ceil(ROTATE_BYTES / (l.N * l.K * 2)))
        W = [torch.randn((l.N, l.K), device=dev, generator=gen).to(torch.bfloat16) for _ in range(R)]
        row = {}
        for mm in (16, 256):
            if mm == 256 and prefill is None:
                continue
            a = torch.randn((mm, l.K), device=dev, generator=gen).to(torch.bfloat16)
            for s in range(5):
                torch.matmul(a, W[s % R].t())
            n = 30
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for s in range(n):
                torch.matmul(a, W[s % R].t())
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / n * 1e3
            ours = per_layer[l.name]["us"] if mm == 16 else prefill["layers"][l.name]["us"]
            row[f"m{mm}"] = {"us": round(us, 2), "TFLOP/s": round(2.0 * mm * l.N * l.K / us / 1e6, 1),
                             "fp4_speedup": round(us / ours, 3)}
        out["layers"][l.name] = row
        del W
        torch.cuda.empty_cache()
    for mm in (16, 256):
        r = [v[f"m{mm}"]["fp4_speedup"] for v in out["layers"].values() if f"m{mm}" in v]
        if r:
            out[f"mean_speedup_m{mm}"] = round(sum(r) / len(r), 3)
            out[f"max_speedup_m{mm}"] = round(max(r), 3)
    return out


def ceilings(torch, dev):
    """Measured ceilings beside the nominal peaks: a 1 GiB device-to-device
    copy (bytes read + written per second) and the BF16 matrix product of the
    vendor library at 8192^3 (hipBLASLt through torch.matmul)."""
    out = {}
    x = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    e0.record()
    for _ in range(n):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    out["copy_GB/s"] = round(2.0 * x.numel() / us / 1e3, 1)
    out["copy_frac_hbm"] = round(out["copy_GB/s"] / HBM_PEAK_GBS, 4)
    del x, y
    gen = torch.Generator(device=dev).manual_seed(5)
    a = torch.randn((8192, 8192), device=dev, generator=gen).to(torch.bfloat16)
    b = torch.randn((8192, 8192), device=dev, generator=gen).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    n = 10
    e0.record()
    for _ in range(n):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    out["bf16_gemm_8192_TFLOP/s"] = round(2.0 * 8192 ** 3 / us / 1e6, 1)
    out["bf16_gemm_frac_mfma"] = round(out["bf16_gemm_8192_TFLOP/s"] / MFMA_BF16_PEAK_TFLOPS, 4)
    out["note"] = "copy: torch copy_ of 1 GiB; gemm: torch.matmul BF16 8192^3 (hipBLASLt)"
    del a, b
    torch.cuda.empty_cache()
    return out


def config_lines(args, F, torch, dev):
    """Roofline fractions of the MXFP4 decode sweep (m = 1, 4, 8, 16 at
    8192 x 28672 and 57344 x 8192) and of the ragged NVFP4 set (m = 1, 7, 33,
    100, 255; N = 1000, 8200; K = 8192).  Weights are random packed bytes on
    the device with valid scale bytes (E8M0 121 .. 129, E4M3 0x18 .. 0x48):
    the timing does not depend on the values; the GPU tests check these
    shapes against the oracle.  t_roof = max(bytes / 8 TB/s, flops /
    2.5 PFLOP/s); frac = t_roof / t."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(91)
    lib = F.lib()
    stream = F._c_vp(torch.cuda.current_stream().cuda_stream)

    def run(N, K, fmt, ms, lo, hi):
        nw, ns = F.repack_size(N, K, fmt)
        R = max(2, math.ceil(ROTATE_BYTES / (nw + ns)))
        copies = [(torch.randint(0, 256, (nw,), dtype=torch.uint8, device=dev, generator=gen),
                   torch.randint(lo, hi + 1, (ns,), dtype=torch.uint8, device=dev, generator=gen)) for _ in range(R)]
        G = 16 if fmt == 0 else 32
        rows = []
        for m in ms:
            a = torch.randn((m, K), device=dev, generator=gen).to(torch.bfloat16)
            c = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
            ws = F.new_workspace(m, N, K, fmt, device=dev)
            wsb = ws.numel() if ws is not None else 0
            argv = [(F._dev_ptr(a), F._dev_ptr(wq), F._dev_ptr(sq), F._dev_ptr(c), m, N, K, fmt, F._dev_ptr(ws), wsb,
                     stream) for wq, sq in copies]

            def call(s_, argv=argv):
                st = lib.fp4_gemm(*argv[s_ % len(argv)])
                if st:
                    F._check(st, "fp4_gemm")
            for s_ in range(5):
                call(s_)
            us = timed(call, max(30, 2 * R))
            b = algorithmic_bytes(m, N, K, G)
            fl = 2.0 * m * N * K
            t_roof = max(b / (HBM_PEAK_GBS * 1e3), fl / (MFMA_BF16_PEAK_TFLOPS * 1e6))
            rows.append({"m": m, "N": N, "K": K, "us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                         "TFLOP/s": round(fl / us / 1e6, 1),
                         "bound": "hbm" if b / (HBM_PEAK_GBS * 1e3) >= fl / (MFMA_BF16_PEAK_TFLOPS * 1e6) else "mfma",
                         "frac": round(t_roof / us, 4)})
        del copies
        torch.cuda.empty_cache()
        return rows

    mx = run(8192, 28672, 1, (1, 4, 8, 16), 121, 129) + run(57344, 8192, 1, (1, 4, 8, 16), 121, 129)
    rg = run(1000, 8192, 0, (1, 7, 33, 100, 255), 0x18, 0x48) + run(8200, 8192, 0, (1, 7, 33, 100, 255), 0x18, 0x48)
    return {"mxfp4_decode": mx, "ragged_nvfp4": rg,
            "note": "frac = max(bytes / 8 TB/s, flops / 2.5 PFLOP/s) / measured time per launch"}


def moe_lines(args, F, torch, synth, dev):
    """Grouped MoE GEMM at 16 and 256 tokens.  The expert weights are random
    packed bytes made on the device (the packed layout is a permutation of
    the codes, so random bytes are random codes; E8M0 scale bytes 121 ..
    129): the timing does not depend on the values, and the parity of these
    shapes is covered by the GPU tests with seeded codes.  Two copies of all
    experts (2 x 1.13 GB) alternate between launches so the 256 MB
    last-level cache cannot serve the weights."""
    E, topk, N, K, fmt = 128, 4, 5760, 2880, 1
    nw, ns = F.repack_size(N, K, fmt)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    copies = []
    for _ in range(2):
        wq = torch.randint(0, 256, (E * nw,), dtype=torch.uint8, device=dev, generator=gen)
        sq = torch.randint(121, 130, (E * ns,), dtype=torch.uint8, device=dev, generator=gen)
        copies.append((wq, sq))
    lib = F.lib()
    stream = F._c_vp(torch.cuda.current_stream().cuda_stream)
    out = {"experts": E, "topk": topk, "N": N, "K": K, "weights": "mxfp4", "activations": "bf16"}
    for T in (16, 256):
        ids, offs, topw = synth.moe_routing(T, topk, E, seed=4242 + T)
        a = torch.randn((T, K), device=dev).to(torch.bfloat16)
        c = torch.empty((T * topk, N), dtype=torch.bfloat16, device=dev)
        ids_d, offs_d, topw_d = (torch.from_numpy(ids).to(dev), torch.from_numpy(offs).to(dev),
                                 torch.from_numpy(topw).to(dev))
        calls = []
        for wq, sq in copies:
            argv = (F._dev_ptr(a), F._dev_ptr(wq), F._dev_ptr(sq), F._dev_ptr(ids_d), F._dev_ptr(offs_d),
                    F._dev_ptr(topw_d), F._dev_ptr(c), T, topk, T * topk, ids.size, E, N, K, fmt, stream)
            calls.append(argv)

        def call(s, calls=calls):
            st = lib.fp4_moe_gemm(*calls[s % 2])
            if st:
                F._check(st, "fp4_moe_gemm")
        for s in range(5):
            call(s)
        torch.cuda.synchronize()
        us = timed(call, args.prefill_launches)
        active = int(np.count_nonzero(np.diff(offs)))
        b = active * (N * K // 2 + N * K // 32) + ids.size * K * 2 + ids.size * N * 2
        fl = 2.0 * ids.size * N * K
        out[f"T{T}"] = {"us": round(us, 2), "active_experts": active, "assignments": int(ids.size),
                        "GB/s": round(b / us / 1e3, 1), "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                        "TFLOP/s": round(fl / us / 1e6, 2)}
    del copies
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.traffic_record:
        rec = traffic_record(*args.traffic_record)
        print(json.dumps({k: rec[k] for k in ("hbm_bytes_per_launch", "algorithmic_bytes_per_launch")}))
        return
    if args.counter_record:
        rec = counter_record(args.counter_record)
        print(f"{len(rec['kernels'])} kernel rows written to {COUNTER_RECORD}")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this GEMM has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mixed_precision_bf16_amd import fp4gemm as F
    from mixed_precision_bf16_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    F.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 268435456 bytes read, 268435456 bytes written")

    t0 = time.time()
    probs = [synth.make_problem(1, si, 0) for si in range(4)]
    layers = [Layer(p, F, torch) for p in probs]
    log(f"inputs ready in {time.time() - t0:.1f}s; rotation copies {[l.R for l in layers]}")
    m = 16
    A = [torch.from_numpy(p.a_bits.view(np.int16)).to(dev).view(torch.bfloat16) for p in probs]
    C = [torch.empty((m, l.N), dtype=torch.bfloat16, device=dev) for l in layers]
    WS = [F.new_workspace(m, l.N, l.K, l.fmt, device=dev) for l in layers]
    calls = [[make_call(F, torch, l, A[i], C[i], r, WS[i]) for r in range(l.R)] for i, l in enumerate(layers)]
    bytes_step = sum(algorithmic_bytes(m, l.N, l.K, l.G) for l in layers)
    dom = 2  # gate_up

    def step(s):
        for i, l in enumerate(layers):
            calls[i][s % l.R]()

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(args.warmup + s)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    # dominant kernel: back-to-back launches (each on the next weight copy)
    dl = layers[dom]
    n_dom = max(args.steps, 4 * dl.R)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(n_dom):
        calls[dom][s % dl.R]()
    e1.record()
    torch.cuda.synchronize()
    dom_us = e0.elapsed_time(e1) / n_dom * 1e3
    # the same launches with events around each one: median and minimum
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dom)]
    for s, (a, b) in enumerate(ev):
        a.record()
        calls[dom][s % dl.R]()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    dom_median, dom_min = per[len(per) // 2], per[0]
    gbs = bytes_step / (ms_step * 1e-3) / 1e9
    dom_bytes = algorithmic_bytes(m, dl.N, dl.K, dl.G)
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9
    log(f"decode step {ms_step * 1e3:.1f} us -> {gbs:.0f} GB/s; gate_up launch {dom_us:.1f} us -> {dom_gbs:.0f} GB/s")

    # per-layer launch times (outside the timed step loop; each layer alone)
    per_layer = {}
    for i, l in enumerate(layers):
        n = max(20, 2 * l.R)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(n):
            calls[i][s % l.R]()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n * 1e3
        b = algorithmic_bytes(m, l.N, l.K, l.G)
        per_layer[l.name] = {"N": l.N, "K": l.K, "us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                             "frac_hbm": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}

    prefill = None
    if not args.no_prefill:
        mp = 256
        rng = np.random.Generator(np.random.PCG64(2_000_000))
        pre = {}
        tot_f, tot_t = 0.0, 0.0
        for i, l in enumerate(layers):
            a = torch.from_numpy(rng.standard_normal((mp, l.K), dtype=np.float32)).to(torch.bfloat16).to(dev)
            c = torch.empty((mp, l.N), dtype=torch.bfloat16, device=dev)
            ws = F.new_workspace(mp, l.N, l.K, l.fmt, device=dev)
            pc = [make_call(F, torch, l, a, c, r, ws) for r in range(l.R)]
            for s in range(5):
                pc[s % l.R]()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = args.prefill_launches
            e0.record()
            for s in range(n):
                pc[s % l.R]()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / n * 1e3
            fl = 2.0 * mp * l.N * l.K
            tot_f += fl
            tot_t += us
            pre[l.name] = {"us": round(us, 2), "TFLOP/s": round(fl / us / 1e6, 1),
                           "frac_mfma": round(fl / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}
        prefill = {"m": mp, "layers": pre, "TFLOP/s": round(tot_f / tot_t / 1e6, 1),
                   "frac_mfma": round(tot_f / tot_t / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                   "peak_TFLOP/s": MFMA_BF16_PEAK_TFLOPS,
                   "note": "weights of the decode layers; A drawn N(0,1) in BF16 with its own seed"}
        log(f"prefill m=256: {prefill['TFLOP/s']} TFLOP/s")

    ceil = None
    if not args.no_blas:
        ceil = ceilings(torch, dev)
        log(f"ceilings: copy {ceil['copy_GB/s']} GB/s, BF16 GEMM 8192^3 {ceil['bf16_gemm_8192_TFLOP/s']} TFLOP/s")

    blas = None
    if not args.no_blas:
        blas = blas_lines(args, torch, layers, per_layer, prefill, dev)
        log("hipBLASLt bf16: fp4 speed-up m=16 mean " + str(blas.get("mean_speedup_m16")) + ", m=256 mean "
            + str(blas.get("mean_speedup_m256")))

    cfg = None
    if not args.no_configs:
        cfg = config_lines(args, F, torch, dev)
        log("mxfp4 decode frac: " + ", ".join(f"m={r['m']} {r['N']}x{r['K']} {r['frac']}" for r in cfg["mxfp4_decode"]))

    fp16 = None
    if not args.no_fp16:
        fp16 = fp16_lines(args, F, torch, layers, A, WS, dev, m)
        log(f"fp16: decode step {fp16['decode_step_us']} us -> {fp16['decode_GB/s']} GB/s; "
            f"prefill m=256 {fp16['prefill_TFLOP/s']} TFLOP/s")

    quant = None
    if not args.no_quantize:
        quant = quantize_lines(args, F, torch, dev)
        log(f"quantize 57344x8192: nvfp4 {quant['nvfp4']['us']} us ({quant['nvfp4']['GB/s']} GB/s), "
            f"mxfp4 {quant['mxfp4']['us']} us ({quant['mxfp4']['GB/s']} GB/s)")

    native = None
    if args.native:
        native = native_lines(args, F, torch, dev)
        log(f"native fp4: prefill m=256 {native['prefill_TFLOP/s']} TFLOP/s, decode m=16 {native['decode_GB/s']} GB/s")

    moe = None
    if not args.no_moe:
        moe = moe_lines(args, F, torch, synth, dev)
        log("moe: " + ", ".join(f"T={t}: {moe[f'T{t}']['us']} us, {moe[f'T{t}']['GB/s']} GB/s"
                                for t in (16, 256)))

    cpu = None if args.no_cpu_baseline else cpu_baseline(probs)

    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode NVFP4 GEMM, m=16, Llama-3-70B layer shapes "
                               "(qkv 10240x8192, o 8192x8192, gate_up 57344x8192, down 8192x28672)",
                   "m": m, "weights": "nvfp4 (E2M1 codes, E4M3 scale per 16)", "activations": "bf16",
                   "accumulate": "fp32", "rotating_weight_copies": {l.name: l.R for l in layers}},
        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "gemm_decode (gate_up, m=16)", "bound": "hbm", "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": dom_bytes, "us_per_launch": round(dom_us, 2), "launches": n_dom,
                     "us_per_launch_median": round(dom_median, 2), "us_per_launch_min": round(dom_min, 2),
                     "traffic": measured_traffic()},
        "layers": per_layer,
        "prefill": prefill,
        "vs_hipblaslt_bf16": blas,
        "measured_ceilings": ceil,
        "other_configs": cfg,
        "fp16": fp16,
        "native": native,
        "moe": moe,
        "quantize": quant,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
