"""Benchmark of the MXFP4 / NVFP4 hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W]

One step runs every row of the hot path once, on seeded synthetic inputs
already resident in HBM:
  tiny   MXFP4 quantize (fp32 256x512) + dequantize + W4A16 GEMV (m=1)
  quant  dynamic MXFP4 quantize of bf16 activations 16384x8192
  gemv   W4A16 decode GEMV, MXFP4 weight 28672x8192, bf16 x at m = 1, 4, 16
         (four copies of the quantized weight are rotated so every call
         streams its weight from HBM, not from the 256 MB Infinity Cache)
  w4a4   MXFP4 quantize of A 8192x8192 + W4A4 GEMM 8192^3 on block-scaled MFMA
  c5     NVFP4 and MXFP4 quantize of W 8192x4096 and X 4096x4096, and the
         W4A16 GEMM Y = X W^T (4096x8192x4096) in each format
Each call is bracketed by HIP events on the stream the library launches on
(torch's current stream).  The JSON line's value is the decode GEMV's
achieved HBM bandwidth at m = 1 (algorithmic bytes / average kernel time);
the W4A4 GEMM TFLOP/s is reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MXFP4 W4A16 GEMV HBM GB/s (% peak); W4A4 GEMM TFLOPS (% MXFP4 MFMA peak)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="", help="comma list of parts to run (tiny,quant,gemv,w4a4,c5)")
    return p.parse_args()


# ---------------------------------------------------------------- byte / flop models
# Algorithmic traffic: what the method must move, each operand once.

def mx_bytes(rows, k):  # packed codes + E8M0 scales
    return rows * k // 2 + rows * k // 32


def nv_bytes(rows, k):  # codes + E4M3 scales + fp32 tensor scale
    return rows * k // 2 + rows * k // 16 + 4


def gemv_bytes(n, k, m):
    return mx_bytes(n, k) + m * k * 2 + m * n * 2


def quant_bytes(rows, k, in_bytes=2):
    return rows * k * in_bytes + mx_bytes(rows, k)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import mxfp4_microscaling_quantization_mxq_amd as mxq
    from mxfp4_microscaling_quantization_mxq_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mxq.capi()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    parts = set(args.only.split(",")) if args.only else {"tiny", "quant", "gemv", "w4a4", "c5"}

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    t_gen = time.time()
    print("generating inputs ...", file=sys.stderr, flush=True)
    ops = []  # (name, callable, bytes, flops)
    bf16 = torch.bfloat16
    if "tiny" in parts:
        w1, x1 = synth.tiny_ref()
        w1d, x1d = to_dev(w1), to_dev(x1)
        q1 = torch.empty((256, 256), dtype=torch.uint8, device=dev)
        s1 = torch.empty((256, 16), dtype=torch.uint8, device=dev)
        y1 = torch.empty((256, 512), dtype=torch.float32, device=dev)
        g1 = torch.empty((1, 256), dtype=bf16, device=dev)
        ops.append(("tiny_quantize_f32", lambda: mxq.quantize(w1d, q1, s1), quant_bytes(256, 512, 4), 0))
        ops.append(("tiny_dequantize_f32", lambda: mxq.dequantize(q1, s1, y=y1),
                    mx_bytes(256, 512) + 256 * 512 * 4, 0))
        ops.append(("tiny_gemv_m1", lambda: mxq.gemv_w4a16(q1, s1, x1d, y=g1), gemv_bytes(256, 512, 1),
                    2 * 256 * 512))
    if "quant" in parts:
        x3 = to_dev(synth.dynamic_quantize())
        q3 = torch.empty((16384, 4096), dtype=torch.uint8, device=dev)
        s3 = torch.empty((16384, 256), dtype=torch.uint8, device=dev)
        ops.append(("quantize_16384x8192_bf16", lambda: mxq.quantize(x3, q3, s3), quant_bytes(16384, 8192), 0))
    if "gemv" in parts:
        n2, k2 = 28672, 8192
        w2, _ = synth.decode_gemv(1)
        w2d = to_dev(w2)
        q2, s2 = mxq.quantize(w2d)
        del w2d, w2
        copies = [(q2, s2)] + [(q2.clone(), s2.clone()) for _ in range(3)]
        xs = {m: to_dev(synth.decode_gemv(m)[1]) for m in (1, 4, 16)}
        ys = {m: torch.empty((m, n2), dtype=bf16, device=dev) for m in (1, 4, 16)}
        rot = {"i": 0}

        def gemv_call(m):
            def f():
                q, s = copies[rot["i"] % 4]
                rot["i"] += 1
                mxq.gemv_w4a16(q, s, xs[m], y=ys[m])
            return f
        for m in (1, 4, 16):
            ops.append((f"gemv_w4a16_m{m}", gemv_call(m), gemv_bytes(n2, k2, m), 2 * m * n2 * k2))
    if "w4a4" in parts:
        a4, b4 = synth.w4a4_operands()
        a4d = to_dev(a4)
        qb4, sb4 = mxq.quantize(to_dev(b4))
        del a4, b4
        qa4 = torch.empty((8192, 4096), dtype=torch.uint8, device=dev)
        sa4 = torch.empty((8192, 256), dtype=torch.uint8, device=dev)
        c4 = torch.empty((8192, 8192), dtype=bf16, device=dev)
        ops.append(("quantize_a_8192x8192_bf16", lambda: mxq.quantize(a4d, qa4, sa4), quant_bytes(8192, 8192), 0))
        ops.append(("gemm_w4a4_8192", lambda: mxq.gemm_w4a4(qa4, sa4, qb4, sb4, c=c4),
                    2 * mx_bytes(8192, 8192) + 8192 * 8192 * 2, 2 * 8192 ** 3))
    if "c5" in parts:
        w5, x5 = synth.nv_vs_mx()
        w5d, x5d = to_dev(w5), to_dev(x5)
        n5, k5, m5 = 8192, 4096, 4096
        bufs = {}
        for nm, rows in (("w", n5), ("x", m5)):
            bufs[nm + "nq"] = torch.empty((rows, k5 // 2), dtype=torch.uint8, device=dev)
            bufs[nm + "ns"] = torch.empty((rows, k5 // 16), dtype=torch.uint8, device=dev)
            bufs[nm + "ng"] = torch.empty(1, dtype=torch.float32, device=dev)
            bufs[nm + "mq"] = torch.empty((rows, k5 // 2), dtype=torch.uint8, device=dev)
            bufs[nm + "ms"] = torch.empty((rows, k5 // 32), dtype=torch.uint8, device=dev)
        y5n = torch.empty((m5, n5), dtype=bf16, device=dev)
        y5m = torch.empty((m5, n5), dtype=bf16, device=dev)
        B = bufs
        gw = {}

        def nv_q_w():
            gw["g"] = mxq.nv_quantize(w5d, None, B["wnq"], B["wns"], B["wng"])[2]
        ops.append(("nv_quantize_w_8192x4096", nv_q_w, n5 * k5 * 2 * 2 + nv_bytes(n5, k5), 0))
        ops.append(("nv_quantize_x_4096x4096", lambda: mxq.nv_quantize(x5d, None, B["xnq"], B["xns"], B["xng"]),
                    m5 * k5 * 2 * 2 + nv_bytes(m5, k5), 0))
        ops.append(("mx_quantize_w_8192x4096", lambda: mxq.quantize(w5d, B["wmq"], B["wms"]),
                    quant_bytes(n5, k5), 0))
        ops.append(("mx_quantize_x_4096x4096", lambda: mxq.quantize(x5d, B["xmq"], B["xms"]),
                    quant_bytes(m5, k5), 0))
        ops.append(("nv_gemm_w4a16_4096x8192x4096", lambda: mxq.nv_gemm(B["wnq"], B["wns"], gw["g"], x5d, y=y5n),
                    nv_bytes(n5, k5) + m5 * k5 * 2 + m5 * n5 * 2, 2 * m5 * n5 * k5))
        ops.append(("mx_gemm_w4a16_4096x8192x4096", lambda: mxq.gemv_w4a16(B["wmq"], B["wms"], x5d, y=y5m),
                    mx_bytes(n5, k5) + m5 * k5 * 2 + m5 * n5 * 2, 2 * m5 * n5 * k5))
    torch.cuda.synchronize()
    print(f"inputs ready in {time.time() - t_gen:.1f}s; warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    nops = len(ops)

    def run_step(evs):
        for i, (_, fn, _, _) in enumerate(ops):
            if evs is not None:
                evs[i][0].record(stream)
            fn()
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        run_step(None)
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(nops)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        run_step(events[st])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_op = {}
    for i, (name, _, nbytes, flops) in enumerate(ops):
        ms = [events[st][i][0].elapsed_time(events[st][i][1]) for st in range(args.steps)]
        avg = float(np.mean(ms))
        per_op[name] = {
            "ms": round(avg, 5),
            "ms_min": round(float(np.min(ms)), 5),
            "GB/s": round(nbytes / avg / 1e6, 1),
            "TFLOP/s": round(flops / avg / 1e9, 1) if flops else None,
            "bytes": nbytes,
            "flops": flops,
        }
        print(f"  {name:34s} {avg * 1e3:10.2f} us  {nbytes / avg / 1e6:9.1f} GB/s"
              + (f"  {flops / avg / 1e9:9.1f} TFLOP/s" if flops else ""), file=sys.stderr, flush=True)

    def roof(name, bound):
        r = per_op[name]
        if bound == "hbm":
            a, p, u = r["GB/s"], HBM_PEAK_GBS, "GB/s"
        elif bound == "mfma_fp4":
            a, p, u = r["TFLOP/s"], FP4_PEAK_TFLOPS, "TFLOP/s"
        else:
            a, p, u = r["TFLOP/s"], BF16_PEAK_TFLOPS, "TFLOP/s"
        out = {"bound": "hbm" if bound == "hbm" else "mfma", "achieved": a, "peak": p, "unit": u,
               "frac": round(a / p, 4), "traffic": traffic_for(name)}
        return out

    rooflines = {}
    for name in per_op:
        if name.startswith("gemm_w4a4"):
            rooflines[name] = roof(name, "mfma_fp4")
        elif "gemm_w4a16_4096" in name:
            rooflines[name] = roof(name, "mfma_bf16")
        else:
            rooflines[name] = roof(name, "hbm")

    head = "gemv_w4a16_m1"
    result = {
        "metric": METRIC,
        "value": per_op[head]["GB/s"] if head in per_op else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1 weights x bf16 activations, fp32 accumulate (W4A4: e2m1 x e2m1)",
        "data": "synthetic (seeded Laplace/normal with outliers; no dataset)",
        "config": {
            "workload": "decode W4A16 GEMV: MXFP4 W 28672x8192 (E8M0/32), x bf16 m=1 (m=4,16 also timed); "
                        "W4A4 GEMM 8192^3; dynamic quantize 16384x8192 bf16; NVFP4 vs MXFP4 W 8192x4096, X 4096x4096",
            "gemv_n": 28672, "gemv_k": 8192, "gemv_m": 1,
        },
        "roofline": rooflines.get(head),
        "secondary": None,
        "rooflines": rooflines,
        "kernels": per_op,
    }
    if "gemm_w4a4_8192" in per_op:
        r = per_op["gemm_w4a4_8192"]
        result["secondary"] = {"metric": "W4A4 GEMM TFLOPS (8192^3, MXFP4 x MXFP4, bf16 out)",
                               "value": r["TFLOP/s"], "unit": "TFLOP/s",
                               "frac_of_mxfp4_peak": round(r["TFLOP/s"] / FP4_PEAK_TFLOPS, 4)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------- traffic from counters

def _src_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mxfp4_microscaling_quantization_mxq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"gemv": ["w4a16.hip", "mxq_device.h"], "w4a4": ["w4a4.hip", "mxq_device.h"],
                  "quantize": ["quant.hip", "mxq_device.h"]}


def traffic_for(name):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE
    (scaled by the copy-kernel calibration), if recorded for the current
    kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    if rec.get("source_digest") != _src_digest(KERNEL_SOURCES[rec["source"]]):
        return None
    return rec.get("bytes")


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline():
    """The oracle (plain C, OpenMP) on a bounded sample of the same workloads."""
    import oracle
    from mxfp4_microscaling_quantization_mxq_amd import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # W4A16 decode GEMV, m = 1, on the first 7168 of the 28672 weight rows
    n_s, k = 7168, 8192
    w, x = synth.decode_gemv(1, n=n_s)
    q, s = oracle.mx_quantize(w)
    t0 = time.perf_counter()
    wd = oracle.mx_dequantize(q, s)
    y, _ = oracle.gemm_nt(oracle.to_f64(x), wd)
    t_gemv = time.perf_counter() - t0
    gemv_gbs = gemv_bytes(n_s, k, 1) / t_gemv / 1e9
    # W4A4 GEMM on a 64 x 512 output sample of the 8192^3 problem
    a, b = synth.w4a4_operands(m=64, n=512)
    qa, sa = oracle.mx_quantize(a)
    qb, sb = oracle.mx_quantize(b)
    t0 = time.perf_counter()
    c, _ = oracle.gemm_nt(oracle.mx_dequantize(qa, sa), oracle.mx_dequantize(qb, sb))
    t_gemm = time.perf_counter() - t0
    gemm_tflops = 2 * 64 * 512 * 8192 / t_gemm / 1e12
    # dynamic quantize on 1024 of the 16384 activation rows
    xq = synth.dynamic_quantize(rows=1024)
    t0 = time.perf_counter()
    oracle.mx_quantize(xq)
    t_q = time.perf_counter() - t0
    return {
        "value": round(gemv_gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"W4A16 GEMV m=1 over {n_s} of 28672 weight rows (k=8192): dequantize + double dot products, "
                  f"{t_gemv:.2f}s; bytes counted as for the GPU kernel",
        "gemm_w4a4_tflops": round(gemm_tflops, 5),
        "gemm_sample": f"64x512 outputs of the 8192^3 W4A4 GEMM, {t_gemm:.2f}s",
        "quantize_GBps": round(quant_bytes(1024, 8192) / t_q / 1e9, 3),
        "quantize_sample": f"1024 of 16384 rows x 8192, {t_q:.2f}s",
        "cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
