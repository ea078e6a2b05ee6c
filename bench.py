"""Benchmark of the MXFP4 / NVFP4 hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only parts] [--no-cpu-baseline]

One step runs every row of the hot path once, on seeded synthetic inputs
already resident in HBM:
  tiny   MXFP4 quantize (fp32 256x512) + dequantize + W4A16 GEMV (m=1)
  quant  dynamic MXFP4 quantize of bf16 activations 16384x8192, plain and
         with the 32-point block Hadamard rotation fused ahead of it; the
         TransFP4 block quantize (rotation, bf16 residual, NVFP4/INT4 choice)
         of the same tensor and its dequantization
  gemv   W4A16 decode GEMV, MXFP4 weight 28672x8192, bf16 x at m = 1, 4, 16
         (and the same weight in NVFP4 at m = 1, 16);
         on the same weight at m = 16: W4A4 (MXFP4 x), W4A8 (MXFP8 x), and
         both from bf16 x quantized inside the GEMM (the small-m kernel)
  w4a4   MXFP4 quantize of A 8192x8192 + W4A4 GEMM 8192^3 on block-scaled MFMA
         (bf16 output, and MXFP4 output quantized in the epilogue); MXFP8
         quantize of the same A + W4A8 GEMM 8192^3 (E4M3 x E2M1 MFMA)
  c5     NVFP4 and MXFP4 quantize of W 8192x4096 and X 4096x4096, and the
         W4A16 GEMM Y = X W^T (4096x8192x4096) in each format
Every HBM-bound op cycles through copies of its operands whose combined size
exceeds the 256 MB Infinity Cache, so each launch streams from HBM.

Timing, all with HIP events on the stream the library launches on (torch's
current stream): K timed steps (ms_per_step = wall time / K; each call also
bracketed by its own event pair), then per op a kernel-rate region of BURST
back-to-back launches per event pair, whose per-launch average is the
kernel's duration used for GB/s, TFLOP/s and the roofline fractions.  The
JSON line's value is the decode GEMV's achieved HBM bandwidth at m = 1
(algorithmic bytes / that duration); the W4A4 GEMM TFLOP/s is beside it.
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
FP8_PEAK_TFLOPS = 5000.0  # dense fp8 MFMA; an E4M3 x E2M1 product issues at this rate
BURST = 16  # launches per event pair in the kernel-rate region
COLD_BYTES = 768 << 20  # rotation set size for HBM-bound ops (3x the 256 MB cache)
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MXFP4 W4A16 GEMV HBM GB/s (% peak); W4A4 GEMM TFLOPS (% MXFP4 MFMA peak)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="",
                   help="comma list of parts to run (tiny,quant,gemv,w4a4,c5; 'copy' adds a 1 GiB device copy "
                        "used to calibrate HBM byte counters)")
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
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path.",
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
    u8 = torch.uint8

    def rotating(sets, call):
        """A callable that runs call(*sets[i]) on the next argument set each
        time: an HBM-bound op cycles through copies whose combined size
        exceeds the 256 MB Infinity Cache, so every launch streams from HBM."""
        st = {"i": 0}

        def f():
            args_ = sets[st["i"] % len(sets)]
            st["i"] += 1
            call(*args_)
        return f

    def ncopies(working_set_bytes):
        return max(1, min(16, -(-COLD_BYTES // working_set_bytes)))

    if "tiny" in parts:
        w1, x1 = synth.tiny_ref()
        w1d, x1d = to_dev(w1), to_dev(x1)
        q1 = torch.empty((256, 256), dtype=u8, device=dev)
        s1 = torch.empty((256, 16), dtype=u8, device=dev)
        y1 = torch.empty((256, 512), dtype=torch.float32, device=dev)
        g1 = torch.empty((1, 256), dtype=bf16, device=dev)
        ops.append(("tiny_quantize_f32", lambda: mxq.quantize(w1d, q1, s1), quant_bytes(256, 512, 4), 0))
        ops.append(("tiny_dequantize_f32", lambda: mxq.dequantize(q1, s1, y=y1),
                    mx_bytes(256, 512) + 256 * 512 * 4, 0))
        ops.append(("tiny_gemv_m1", lambda: mxq.gemv_w4a16(q1, s1, x1d, y=g1), gemv_bytes(256, 512, 1),
                    2 * 256 * 512))
    if "quant" in parts:
        x3 = to_dev(synth.dynamic_quantize())
        n3 = ncopies(quant_bytes(16384, 8192))
        sets = [(x3 if c == 0 else x3.clone(), torch.empty((16384, 4096), dtype=u8, device=dev),
                 torch.empty((16384, 256), dtype=u8, device=dev)) for c in range(n3)]
        ops.append(("quantize_16384x8192_bf16", rotating(sets, lambda x, q, s: mxq.quantize(x, q, s)),
                    quant_bytes(16384, 8192), 0))
        # rotated MXFP4 (32-point block Hadamard fused ahead of the quantizer)
        ops.append(("quantize_hadamard32_16384x8192_bf16",
                    rotating(sets, lambda x, q, s: mxq.quantize_hadamard(x, 32, q, s)), quant_bytes(16384, 8192), 0))
        # TransFP4 blocks: tensor-scale pass + quantize pass (x read twice),
        # then the dequantization back to bf16
        ntf = 16384 * 8192
        tsets = [(x, torch.empty((16384, 4096), dtype=u8, device=dev), torch.empty((16384, 512), dtype=u8, device=dev),
                  torch.empty((16384, 256), dtype=u8, device=dev), torch.empty((16384, 256), dtype=bf16, device=dev),
                  torch.empty(1, dtype=torch.float32, device=dev)) for x, _, _ in sets]
        tf4_bytes = ntf // 2 + ntf // 16 + ntf // 32 + ntf // 16  # codes, E4M3, meta, bf16 residual
        ops.append(("transfp4_quantize_16384x8192_bf16",
                    rotating(tsets, lambda x, q, s, m, r, g: mxq.transfp4_quantize(x, None, q, s, m, r, g)),
                    2 * 2 * ntf + tf4_bytes, 0))
        ydq = [torch.empty((16384, 8192), dtype=bf16, device=dev) for _ in tsets]
        for (x, q, s_, m, r, g) in tsets:
            mxq.transfp4_quantize(x, None, q, s_, m, r, g)
        ops.append(("transfp4_dequantize_16384x8192_bf16",
                    rotating([(q, s_, m, r, g, y) for (x, q, s_, m, r, g), y in zip(tsets, ydq)],
                             lambda q, s_, m, r, g, y: mxq.transfp4_dequantize(q, s_, m, r, g, y=y)),
                    tf4_bytes + 2 * ntf, 0))
    if "gemv" in parts:
        n2, k2 = 28672, 8192
        w2, _ = synth.decode_gemv(1)
        w2d = to_dev(w2)
        q2, s2 = mxq.quantize(w2d)
        del w2d
        nc = ncopies(mx_bytes(n2, k2))
        copies = [(q2, s2)] + [(q2.clone(), s2.clone()) for _ in range(nc - 1)]
        for m in (1, 4, 16, 64):
            xm = to_dev(synth.decode_gemv(m)[1])
            ym = torch.empty((m, n2), dtype=bf16, device=dev)
            ops.append((f"gemv_w4a16_m{m}",
                        rotating([(q, s, xm, ym) for q, s in copies], lambda q, s, x, y: mxq.gemv_w4a16(q, s, x, y=y)),
                        gemv_bytes(n2, k2, m), 2 * m * n2 * k2))
        # the same weight in NVFP4 (E4M3 per 16 + fp32 tensor scale)
        qn2, sn2, gn2 = mxq.nv_quantize(to_dev(w2))
        del w2
        ncn = ncopies(nv_bytes(n2, k2))
        ncopies_nv = [(qn2, sn2)] + [(qn2.clone(), sn2.clone()) for _ in range(ncn - 1)]
        for m in (1, 16, 64):
            xm = to_dev(synth.decode_gemv(m)[1])
            ym = torch.empty((m, n2), dtype=bf16, device=dev)
            ops.append((f"nv_gemv_w4a16_m{m}",
                        rotating([(q, s) for q, s in ncopies_nv],
                                 lambda q, s, x=xm, y=ym: mxq.nv_gemm(q, s, gn2, x, y=y)),
                        nv_bytes(n2, k2) + m * k2 * 2 + m * n2 * 2, 2 * m * n2 * k2))
        # decode-sized W4A4 / W4A8 on the same weight (the small-m kernel:
        # the weight stream bounds it), and W4A4 straight from bf16
        # activations with their quantization fused into the GEMM
        x16 = to_dev(synth.decode_gemv(16)[1])
        qx16, sx16 = mxq.quantize(x16)
        qx8, sx8 = mxq.quantize_fp8(x16)
        y16 = torch.empty((16, n2), dtype=bf16, device=dev)
        out16 = 16 * n2 * 2
        ops.append(("decode_w4a4_m16", rotating([(q, s) for q, s in copies],
                                                lambda q, s: mxq.gemm_w4a4(qx16, sx16, q, s, c=y16)),
                    mx_bytes(n2, k2) + mx_bytes(16, k2) + out16, 2 * 16 * n2 * k2))
        ops.append(("decode_w4a8_m16", rotating([(q, s) for q, s in copies],
                                                lambda q, s: mxq.gemm_w4a8(qx8, sx8, q, s, c=y16)),
                    mx_bytes(n2, k2) + 16 * k2 + 16 * k2 // 32 + out16, 2 * 16 * n2 * k2))
        ops.append(("decode_w4a4_dynamic_m16", rotating([(q, s) for q, s in copies],
                                                        lambda q, s: mxq.gemm_w4a4_dynamic(x16, q, s, c=y16)),
                    mx_bytes(n2, k2) + 16 * k2 * 2 + out16, 2 * 16 * n2 * k2))
        ops.append(("decode_w4a8_dynamic_m16", rotating([(q, s) for q, s in copies],
                                                        lambda q, s: mxq.gemm_w4a8_dynamic(x16, q, s, c=y16)),
                    mx_bytes(n2, k2) + 16 * k2 * 2 + out16, 2 * 16 * n2 * k2))
    if "w4a4" in parts:
        a4, b4 = synth.w4a4_operands()
        a4d = to_dev(a4)
        qb4, sb4 = mxq.quantize(to_dev(b4))
        del a4, b4
        qa4 = torch.empty((8192, 4096), dtype=u8, device=dev)
        sa4 = torch.empty((8192, 256), dtype=u8, device=dev)
        c4 = torch.empty((8192, 8192), dtype=bf16, device=dev)
        na = ncopies(quant_bytes(8192, 8192))
        sets = [(a4d if c == 0 else a4d.clone(), qa4 if c == 0 else torch.empty_like(qa4),
                 sa4 if c == 0 else torch.empty_like(sa4)) for c in range(na)]
        ops.append(("quantize_a_8192x8192_bf16", rotating(sets, lambda x, q, s: mxq.quantize(x, q, s)),
                    quant_bytes(8192, 8192), 0))
        # the GEMM is compute-bound (its 68 MB of operands may stay in the cache)
        ops.append(("gemm_w4a4_8192", lambda: mxq.gemm_w4a4(qa4, sa4, qb4, sb4, c=c4),
                    2 * mx_bytes(8192, 8192) + 8192 * 8192 * 2, 2 * 8192 ** 3))
        # the same product with the MXFP4 quantization of its output fused
        # into the epilogue (the next layer's activations, no bf16 round trip)
        cq4 = torch.empty((8192, 4096), dtype=u8, device=dev)
        cs4 = torch.empty((8192, 256), dtype=u8, device=dev)
        ops.append(("gemm_w4a4_8192_mxfp4_out", lambda: mxq.gemm_w4a4_quant(qa4, sa4, qb4, sb4, cq4, cs4),
                    3 * mx_bytes(8192, 8192), 2 * 8192 ** 3))
        # MXFP8 activations (E4M3 + E8M0 per 32) against the same MXFP4 weights
        qa8 = torch.empty((8192, 8192), dtype=u8, device=dev)
        sa8 = torch.empty((8192, 256), dtype=u8, device=dev)
        sets8 = [(a4d if c == 0 else sets[c][0], qa8 if c == 0 else torch.empty_like(qa8),
                  sa8 if c == 0 else torch.empty_like(sa8)) for c in range(na)]
        ops.append(("quantize_fp8_a_8192x8192_bf16", rotating(sets8, lambda x, q, s: mxq.quantize_fp8(x, q, s)),
                    8192 * 8192 * 3 + 8192 * 256, 0))
        ops.append(("gemm_w4a8_8192", lambda: mxq.gemm_w4a8(qa8, sa8, qb4, sb4, c=c4),
                    8192 * 8192 + 8192 * 256 + mx_bytes(8192, 8192) + 8192 * 8192 * 2, 2 * 8192 ** 3))
    if "c5" in parts:
        w5, x5 = synth.nv_vs_mx()
        w5d, x5d = to_dev(w5), to_dev(x5)
        n5, k5, m5 = 8192, 4096, 4096
        del w5, x5

        def qsets(src, rows, blk):
            nb = ncopies(rows * k5 * 2 + rows * k5 // 2 + rows * k5 // blk)
            return [(src if c == 0 else src.clone(), torch.empty((rows, k5 // 2), dtype=u8, device=dev),
                     torch.empty((rows, k5 // blk), dtype=u8, device=dev),
                     torch.empty(1, dtype=torch.float32, device=dev)) for c in range(nb)]
        nvw, nvx = qsets(w5d, n5, 16), qsets(x5d, m5, 16)
        mxw, mxx = qsets(w5d, n5, 32), qsets(x5d, m5, 32)

        def nvq(x, q, s, g):
            mxq.nv_quantize(x, None, q, s, g)

        def mxqz(x, q, s, g):
            mxq.quantize(x, q, s)
        ops.append(("nv_quantize_w_8192x4096", rotating(nvw, nvq), n5 * k5 * 2 * 2 + nv_bytes(n5, k5), 0))
        ops.append(("nv_quantize_x_4096x4096", rotating(nvx, nvq), m5 * k5 * 2 * 2 + nv_bytes(m5, k5), 0))
        ops.append(("mx_quantize_w_8192x4096", rotating(mxw, mxqz), quant_bytes(n5, k5), 0))
        ops.append(("mx_quantize_x_4096x4096", rotating(mxx, mxqz), quant_bytes(m5, k5), 0))
        y5n = torch.empty((m5, n5), dtype=bf16, device=dev)
        y5m = torch.empty((m5, n5), dtype=bf16, device=dev)
        _, wnq, wns, wng = nvw[0]
        _, wmq, wms, _ = mxw[0]
        mxq.nv_quantize(w5d, None, wnq, wns, wng)
        ops.append(("nv_gemm_w4a16_4096x8192x4096", lambda: mxq.nv_gemm(wnq, wns, wng, x5d, y=y5n),
                    nv_bytes(n5, k5) + m5 * k5 * 2 + m5 * n5 * 2, 2 * m5 * n5 * k5))
        ops.append(("mx_gemm_w4a16_4096x8192x4096", lambda: mxq.gemv_w4a16(wmq, wms, x5d, y=y5m),
                    mx_bytes(n5, k5) + m5 * k5 * 2 + m5 * n5 * 2, 2 * m5 * n5 * k5))
    if "copy" in parts:
        # a plain device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # counters calibrate the HBM byte counts of the other kernels
        csrc = torch.empty(1 << 30, dtype=u8, device=dev)
        cdst = torch.empty_like(csrc)
        csrc.fill_(1)
        ops.append(("copy_1GiB", lambda: cdst.copy_(csrc), 2 << 30, 0))
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
    # timed region 1: K steps, one pass of the hot path each; every call is
    # also bracketed by its own pair of events (single-launch times)
    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(nops)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        run_step(events[st])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # timed region 2: per op, BURST back-to-back launches between one pair of
    # events; elapsed / BURST is the kernel's average launch duration (inter-
    # launch gaps included), free of the few microseconds that an event pair
    # adds around a single short launch.  This is the figure the rooflines use.
    burst = {}
    for i, (name, fn, _, _) in enumerate(ops):
        reps = []
        for _ in range(max(1, args.steps // 4)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(BURST):
                fn()
            e1.record(stream)
            e1.synchronize()
            reps.append(e0.elapsed_time(e1) / BURST)
        burst[name] = float(np.median(reps))
    per_op = {}
    for i, (name, _, nbytes, flops) in enumerate(ops):
        ms = [events[st][i][0].elapsed_time(events[st][i][1]) for st in range(args.steps)]
        avg = burst[name]
        per_op[name] = {
            "ms": round(avg, 5),
            "ms_single_median": round(float(np.median(ms)), 5),
            "ms_single_min": round(float(np.min(ms)), 5),
            "GB/s": round(nbytes / avg / 1e6, 1),
            "TFLOP/s": round(flops / avg / 1e9, 1) if flops else None,
            "bytes": nbytes,
            "flops": flops,
        }
        print(f"  {name:34s} {avg * 1e3:10.2f} us (single {np.median(ms) * 1e3:8.2f})  {nbytes / avg / 1e6:9.1f} GB/s"
              + (f"  {flops / avg / 1e9:9.1f} TFLOP/s" if flops else ""), file=sys.stderr, flush=True)

    def roof(name, bound):
        r = per_op[name]
        if bound == "hbm":
            a, p, u = r["GB/s"], HBM_PEAK_GBS, "GB/s"
        elif bound == "mfma_fp4":
            a, p, u = r["TFLOP/s"], FP4_PEAK_TFLOPS, "TFLOP/s"
        elif bound == "mfma_fp8":
            a, p, u = r["TFLOP/s"], FP8_PEAK_TFLOPS, "TFLOP/s"
        else:
            a, p, u = r["TFLOP/s"], BF16_PEAK_TFLOPS, "TFLOP/s"
        out = {"bound": "hbm" if bound == "hbm" else "mfma", "achieved": a, "peak": p, "unit": u,
               "frac": round(a / p, 4), "traffic": traffic_for(name)}
        return out

    rooflines = {}
    for name in per_op:
        if name.startswith("gemm_w4a4"):  # both output kinds
            rooflines[name] = roof(name, "mfma_fp4")
        elif name.startswith("gemm_w4a8"):
            rooflines[name] = roof(name, "mfma_fp8")
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


KERNEL_SOURCES = {"gemv": ["w4a16.hip", "mxq_device.h"], "w4a4": ["w4a4.hip", "mxq_device.h", "mxq_gemm_common.h"],
                  "w4a8": ["w4a8.hip", "mxq_device.h", "mxq_gemm_common.h"], "quantize": ["quant.hip", "mxq_device.h"],
                  "skinny": ["gemm_skinny.hip", "mxq_device.h", "mxq_gemm_common.h"]}


def traffic_for(name):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE
    (scaled by the copy-kernel calibration), if recorded in
    profiles/hbm_bytes_fetch_write_size.txt for the current kernel source;
    else None."""
    path = os.path.join(ROOT, "profiles", "hbm_bytes_fetch_write_size.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for ln in f:
            parts = ln.split()
            if len(parts) != 5 or parts[0] != "record" or parts[1] != name:
                continue
            kv = dict(p.split("=", 1) for p in parts[2:])
            src = KERNEL_SOURCES.get(kv.get("source"))
            if src is None or kv.get("digest") != _src_digest(src):
                return None
            return int(kv["bytes"])
    return None


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline():
    """The oracle (plain C, OpenMP) on a bounded sample of the same workloads:
    the full decode GEMV (m = 1) repeated for about 8 s, a 1024 x 1024 output
    block of the W4A4 GEMM, and the full dynamic quantize."""
    import oracle
    from mxfp4_microscaling_quantization_mxq_amd import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n2, k2 = 28672, 8192
    w, x = synth.decode_gemv(1)
    q, s = oracle.mx_quantize(w)
    del w
    xd = oracle.to_f64(x)
    reps, t_gemv = 0, 0.0
    while t_gemv < 8.0 and reps < 50:
        t0 = time.perf_counter()
        wd = oracle.mx_dequantize(q, s)
        oracle.gemm_nt(xd, wd)
        t_gemv += time.perf_counter() - t0
        reps += 1
        del wd
    gemv_gbs = reps * gemv_bytes(n2, k2, 1) / t_gemv / 1e9
    a, b = synth.w4a4_operands(m=1024, n=1024)
    qa, sa = oracle.mx_quantize(a)
    qb, sb = oracle.mx_quantize(b)
    t0 = time.perf_counter()
    oracle.gemm_nt(oracle.mx_dequantize(qa, sa), oracle.mx_dequantize(qb, sb))
    t_gemm = time.perf_counter() - t0
    gemm_tflops = 2 * 1024 * 1024 * 8192 / t_gemm / 1e12
    xq = synth.dynamic_quantize()
    t0 = time.perf_counter()
    oracle.mx_quantize(xq)
    t_q = time.perf_counter() - t0
    return {
        "value": round(gemv_gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"decode W4A16 GEMV m=1 on the full 28672x8192 weight, {reps} runs in {t_gemv:.1f}s "
                  f"(dequantize to double + double dot products); bytes counted as for the GPU kernel",
        "gemm_w4a4_tflops": round(gemm_tflops, 5),
        "gemm_sample": f"1024x1024 outputs of the 8192^3 W4A4 GEMM (k = 8192), {t_gemm:.2f}s",
        "quantize_GBps": round(quant_bytes(16384, 8192) / t_q / 1e9, 3),
        "quantize_sample": f"full 16384x8192 bf16 dynamic quantize, {t_q:.2f}s",
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
