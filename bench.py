"""Benchmark of the MXFP4 / NVFP4 hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--singles N] [--only parts] [--ops names]
                [--no-cpu-baseline] [--no-ceilings] [--no-metrics]

One step runs every row of the hot path once, on seeded synthetic inputs
already resident in HBM:
  tiny   MXFP4 quantize (fp32 256x512) + dequantize + W4A16 GEMV (m=1)
  quant  dynamic MXFP4 quantize of bf16 activations 16384x8192, plain and
         with the 32-point block Hadamard rotation fused ahead of it; the
         TransFP4 block quantize (rotation, bf16 residual, NVFP4/INT4 choice)
         of the same tensor and its dequantization
  gemv   W4A16 decode GEMV, MXFP4 weight 28672x8192, bf16 x at m = 1, 4, 16
         (and 64; the same weight in NVFP4 at m = 1, 16, 64); on the same
         weight at m = 16: W4A4 (MXFP4 x), W4A8 (MXFP8 x), and both from bf16
         x quantized inside the GEMM (the small-m kernel)
  w4a4   MXFP4 quantize of A 8192x8192 + W4A4 GEMM 8192^3 on block-scaled MFMA
         (bf16 output, and MXFP4 output quantized in the epilogue); MXFP8
         quantize of the same A + W4A8 GEMM 8192^3 (E4M3 x E2M1 MFMA)
  c5     NVFP4 and MXFP4 quantize of W 8192x4096 and X 4096x4096, and the
         W4A16 GEMM Y = X W^T (4096x8192x4096) in each format
Every HBM-bound op cycles through copies of its operands whose combined size
exceeds the 256 MB Infinity Cache, so each launch streams from HBM.

Timing, with HIP events on the stream the library launches on (torch's
current stream):
  1. K timed steps of the whole path, bracketed by a synchronize on both
     sides: ms_per_step.
  2. Per op, N (default 50) launches queued back to back, each between its
     own event pair: the median is the op's single-launch duration (an event
     pair adds the time the command processor takes to retire the marker
     packets around one launch, a few microseconds).
  3. Per op, bursts of 16 back-to-back launches between one event pair: the
     per-launch average is the kernel's steady-state duration.  The roofline
     figures (GB/s, TFLOP/s, fractions of the datasheet peak and of the
     measured ceiling) use it; both durations are in the JSON line.
The on-box ceilings (a pure streaming read of the decode weight's size, a
pure streaming write of the largest output, the fp4 and bf16 MFMA issue
rates with the shader clock they ran at) come from the measurement kernels
in libmxq_ceiling.so; an HBM op is held to the time the pure read of its
read bytes plus the pure write of its written bytes would take.  After timing, the quality
metrics (NMSE, cosine; host, float64) of the tiny reference and of the
NVFP4-vs-MXFP4 tensors and products are computed from the GPU's outputs.
The JSON line's value is the decode GEMV's achieved HBM bandwidth at m = 1.
"""
from __future__ import annotations

import argparse
import ctypes
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
BF16_PEAK_TFLOPS = 2500.0
PEAKS = {"hbm": HBM_PEAK_GBS, "fp4": FP4_PEAK_TFLOPS, "fp8": FP8_PEAK_TFLOPS, "bf16": BF16_PEAK_TFLOPS}
BURST = 16  # launches per event pair in the burst region
COLD_BYTES = 768 << 20  # rotation set size for HBM-bound ops (3x the 256 MB cache)
METRIC = "MXFP4 W4A16 GEMV HBM GB/s (% peak); W4A4 GEMM TFLOPS (% MXFP4 MFMA peak)"
HEAD = "gemv_w4a16_m1"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--singles", type=int, default=50, help="single launches per op (median)")
    p.add_argument("--bursts", type=int, default=5, help="bursts of 16 launches per op (median)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceilings", action="store_true")
    p.add_argument("--no-metrics", action="store_true")
    p.add_argument("--only", default="",
                   help="comma list of parts to run (tiny,quant,gemv,w4a4,c5; 'copy' adds a 1 GiB device copy "
                        "used to calibrate HBM byte counters)")
    p.add_argument("--ops", default="", help="comma list of op-name prefixes to time (default: all)")
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
    ops = []  # (name, callable, bytes, flops, bound)
    keep = {}  # GPU tensors the quality metrics read after timing
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
        ops.append(("tiny_quantize_f32", lambda: mxq.quantize(w1d, q1, s1), quant_bytes(256, 512, 4), 0, "hbm",
                    mx_bytes(256, 512)))
        ops.append(("tiny_dequantize_f32", lambda: mxq.dequantize(q1, s1, y=y1),
                    mx_bytes(256, 512) + 256 * 512 * 4, 0, "hbm", 256 * 512 * 4))
        ops.append(("tiny_gemv_m1", lambda: mxq.gemv_w4a16(q1, s1, x1d, y=g1), gemv_bytes(256, 512, 1),
                    2 * 256 * 512, "hbm", 256 * 2))
        keep["tiny"] = (w1, x1, y1, g1)
    if "quant" in parts:
        x3 = to_dev(synth.dynamic_quantize())
        n3 = ncopies(quant_bytes(16384, 8192))
        sets = [(x3 if c == 0 else x3.clone(), torch.empty((16384, 4096), dtype=u8, device=dev),
                 torch.empty((16384, 256), dtype=u8, device=dev)) for c in range(n3)]
        ops.append(("quantize_16384x8192_bf16", rotating(sets, lambda x, q, s: mxq.quantize(x, q, s)),
                    quant_bytes(16384, 8192), 0, "hbm", mx_bytes(16384, 8192)))
        # rotated MXFP4 (32-point block Hadamard fused ahead of the quantizer)
        ops.append(("quantize_hadamard32_16384x8192_bf16",
                    rotating(sets, lambda x, q, s: mxq.quantize_hadamard(x, 32, q, s)), quant_bytes(16384, 8192), 0,
                    "hbm", mx_bytes(16384, 8192)))
        # TransFP4 blocks: tensor-scale pass + quantize pass (x read twice),
        # then the dequantization back to bf16
        ntf = 16384 * 8192
        tsets = [(x, torch.empty((16384, 4096), dtype=u8, device=dev), torch.empty((16384, 512), dtype=u8, device=dev),
                  torch.empty((16384, 256), dtype=u8, device=dev), torch.empty((16384, 256), dtype=bf16, device=dev),
                  torch.empty(1, dtype=torch.float32, device=dev)) for x, _, _ in sets]
        tf4_bytes = ntf // 2 + ntf // 16 + ntf // 32 + ntf // 16  # codes, E4M3, meta, bf16 residual
        ops.append(("transfp4_quantize_16384x8192_bf16",
                    rotating(tsets, lambda x, q, s, m, r, g: mxq.transfp4_quantize(x, None, q, s, m, r, g)),
                    2 * 2 * ntf + tf4_bytes, 0, "hbm", tf4_bytes))
        ydq = [torch.empty((16384, 8192), dtype=bf16, device=dev) for _ in tsets]
        for (x, q, s_, m, r, g) in tsets:
            mxq.transfp4_quantize(x, None, q, s_, m, r, g)
        ops.append(("transfp4_dequantize_16384x8192_bf16",
                    rotating([(q, s_, m, r, g, y) for (x, q, s_, m, r, g), y in zip(tsets, ydq)],
                             lambda q, s_, m, r, g, y: mxq.transfp4_dequantize(q, s_, m, r, g, y=y)),
                    tf4_bytes + 2 * ntf, 0, "hbm", 2 * ntf))
        # MXFP4 dequantize of the same tensor back to bf16 (codes and scales
        # of the plain quantize above)
        dsets = []
        for (x, q, s_), y in zip(sets, ydq):
            q2, s2 = torch.empty_like(q), torch.empty_like(s_)
            mxq.quantize(x, q2, s2)
            dsets.append((q2, s2, y))
        ops.append(("dequantize_16384x8192_bf16", rotating(dsets, lambda q, s_, y: mxq.dequantize(q, s_, y=y)),
                    ntf // 2 + ntf // 32 + 2 * ntf, 0, "hbm", 2 * ntf))
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
                        gemv_bytes(n2, k2, m), 2 * m * n2 * k2, "hbm", 2 * m * n2))
        # the same weight in NVFP4 (E4M3 per 16 + fp32 tensor scale)
        qn2, sn2, gn2 = mxq.nv_quantize(to_dev(w2))
        del w2
        ncn = ncopies(nv_bytes(n2, k2))
        ncopies_nv = [(qn2, sn2)] + [(qn2.clone(), sn2.clone()) for _ in range(ncn - 1)]
        for m in (1, 4, 16, 64):
            xm = to_dev(synth.decode_gemv(m)[1])
            ym = torch.empty((m, n2), dtype=bf16, device=dev)
            ops.append((f"nv_gemv_w4a16_m{m}",
                        rotating([(q, s) for q, s in ncopies_nv],
                                 lambda q, s, x=xm, y=ym: mxq.nv_gemm(q, s, gn2, x, y=y)),
                        nv_bytes(n2, k2) + m * k2 * 2 + m * n2 * 2, 2 * m * n2 * k2, "hbm", 2 * m * n2))
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
                    mx_bytes(n2, k2) + mx_bytes(16, k2) + out16, 2 * 16 * n2 * k2, "hbm", out16))
        ops.append(("decode_w4a8_m16", rotating([(q, s) for q, s in copies],
                                                lambda q, s: mxq.gemm_w4a8(qx8, sx8, q, s, c=y16)),
                    mx_bytes(n2, k2) + 16 * k2 + 16 * k2 // 32 + out16, 2 * 16 * n2 * k2, "hbm", out16))
        ops.append(("decode_w4a4_dynamic_m16", rotating([(q, s) for q, s in copies],
                                                        lambda q, s: mxq.gemm_w4a4_dynamic(x16, q, s, c=y16)),
                    mx_bytes(n2, k2) + 16 * k2 * 2 + out16, 2 * 16 * n2 * k2, "hbm", out16))
        ops.append(("decode_w4a8_dynamic_m16", rotating([(q, s) for q, s in copies],
                                                        lambda q, s: mxq.gemm_w4a8_dynamic(x16, q, s, c=y16)),
                    mx_bytes(n2, k2) + 16 * k2 * 2 + out16, 2 * 16 * n2 * k2, "hbm", out16))
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
                    quant_bytes(8192, 8192), 0, "hbm", mx_bytes(8192, 8192)))
        # the GEMM is compute-bound (its 68 MB of operands may stay in the cache)
        ops.append(("gemm_w4a4_8192", lambda: mxq.gemm_w4a4(qa4, sa4, qb4, sb4, c=c4),
                    2 * mx_bytes(8192, 8192) + 8192 * 8192 * 2, 2 * 8192 ** 3, "fp4"))
        # the same product with the MXFP4 quantization of its output fused
        # into the epilogue (the next layer's activations, no bf16 round trip)
        cq4 = torch.empty((8192, 4096), dtype=u8, device=dev)
        cs4 = torch.empty((8192, 256), dtype=u8, device=dev)
        ops.append(("gemm_w4a4_8192_mxfp4_out", lambda: mxq.gemm_w4a4_quant(qa4, sa4, qb4, sb4, cq4, cs4),
                    3 * mx_bytes(8192, 8192), 2 * 8192 ** 3, "fp4"))
        # MXFP8 activations (E4M3 + E8M0 per 32) against the same MXFP4 weights
        qa8 = torch.empty((8192, 8192), dtype=u8, device=dev)
        sa8 = torch.empty((8192, 256), dtype=u8, device=dev)
        sets8 = [(a4d if c == 0 else sets[c][0], qa8 if c == 0 else torch.empty_like(qa8),
                  sa8 if c == 0 else torch.empty_like(sa8)) for c in range(na)]
        ops.append(("quantize_fp8_a_8192x8192_bf16", rotating(sets8, lambda x, q, s: mxq.quantize_fp8(x, q, s)),
                    8192 * 8192 * 3 + 8192 * 256, 0, "hbm", 8192 * 8192 + 8192 * 256))
        ops.append(("gemm_w4a8_8192", lambda: mxq.gemm_w4a8(qa8, sa8, qb4, sb4, c=c4),
                    8192 * 8192 + 8192 * 256 + mx_bytes(8192, 8192) + 8192 * 8192 * 2, 2 * 8192 ** 3, "fp8"))
    if "c5" in parts:
        w5, x5 = synth.nv_vs_mx()
        w5d, x5d = to_dev(w5), to_dev(x5)
        n5, k5, m5 = 8192, 4096, 4096

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
        ops.append(("nv_quantize_w_8192x4096", rotating(nvw, nvq), n5 * k5 * 2 * 2 + nv_bytes(n5, k5), 0, "hbm",
                    nv_bytes(n5, k5)))
        ops.append(("nv_quantize_x_4096x4096", rotating(nvx, nvq), m5 * k5 * 2 * 2 + nv_bytes(m5, k5), 0, "hbm",
                    nv_bytes(m5, k5)))
        ops.append(("mx_quantize_w_8192x4096", rotating(mxw, mxqz), quant_bytes(n5, k5), 0, "hbm", mx_bytes(n5, k5)))
        ops.append(("mx_quantize_x_4096x4096", rotating(mxx, mxqz), quant_bytes(m5, k5), 0, "hbm", mx_bytes(m5, k5)))
        y5n = torch.empty((m5, n5), dtype=bf16, device=dev)
        y5m = torch.empty((m5, n5), dtype=bf16, device=dev)
        _, wnq, wns, wng = nvw[0]
        _, wmq, wms, _ = mxw[0]
        mxq.nv_quantize(w5d, None, wnq, wns, wng)
        mxq.quantize(w5d, wmq, wms)
        ops.append(("nv_gemm_w4a16_4096x8192x4096", lambda: mxq.nv_gemm(wnq, wns, wng, x5d, y=y5n),
                    nv_bytes(n5, k5) + m5 * k5 * 2 + m5 * n5 * 2, 2 * m5 * n5 * k5, "bf16"))
        ops.append(("mx_gemm_w4a16_4096x8192x4096", lambda: mxq.gemv_w4a16(wmq, wms, x5d, y=y5m),
                    mx_bytes(n5, k5) + m5 * k5 * 2 + m5 * n5 * 2, 2 * m5 * n5 * k5, "bf16"))
        keep["c5"] = (w5, x5, w5d, x5d, y5m, y5n)
    if "copy" in parts:
        # a plain device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # counters calibrate the HBM byte counts of the other kernels
        csrc = torch.empty(1 << 30, dtype=u8, device=dev)
        cdst = torch.empty_like(csrc)
        csrc.fill_(1)
        ops.append(("copy_1GiB", lambda: cdst.copy_(csrc), 2 << 30, 0, "hbm", 1 << 30))
    if args.ops:
        pref = tuple(args.ops.split(","))
        ops = [o for o in ops if o[0].startswith(pref)]
    torch.cuda.synchronize()
    print(f"inputs ready in {time.time() - t_gen:.1f}s; warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def run_step():
        for op in ops:
            op[1]()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    # 1. K steps of the whole path
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"{args.steps} steps: {wall / args.steps * 1e3:.3f} ms per step", file=sys.stderr, flush=True)

    # 2 and 3: per op, single launches and bursts
    per_op = {}
    for op in ops:
        # (name, fn, bytes, flops, bound[, bytes written]): an HBM op's bytes
        # count reads and writes; the written part prices its ceiling
        name, fn, nbytes, flops, bound = op[:5]
        wbytes = op[5] if len(op) > 5 else 0
        fn()
        fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.singles)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        single = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
        reps = []
        for _ in range(args.bursts):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(BURST):
                fn()
            e1.record(stream)
            e1.synchronize()
            reps.append(e0.elapsed_time(e1) / BURST)
        ms = float(np.median(reps))
        per_op[name] = {
            "ms": round(ms, 5),
            "ms_single_median": round(float(np.median(single)), 5),
            "ms_single_min": round(float(single.min()), 5),
            "singles": len(single),
            "GB/s": round(nbytes / ms / 1e6, 1),
            "TFLOP/s": round(flops / ms / 1e9, 1) if flops else None,
            "bytes": nbytes,
            "bytes_written": wbytes,
            "flops": flops,
            "bound": bound,
        }
        print(f"  {name:36s} {ms * 1e3:9.2f} us (single median {np.median(single) * 1e3:8.2f}, "
              f"min {single.min() * 1e3:8.2f})  {nbytes / ms / 1e6:9.1f} GB/s"
              + (f"  {flops / ms / 1e9:9.1f} TFLOP/s" if flops else ""), file=sys.stderr, flush=True)

    ceil = None if args.no_ceilings else measure_ceilings(torch, dev, stream)

    def roof(name):
        r = per_op[name]
        bound = r["bound"]
        a = r["GB/s"] if bound == "hbm" else r["TFLOP/s"]
        p = PEAKS[bound]
        out = {"bound": "hbm" if bound == "hbm" else "mfma", "achieved": a, "peak": p,
               "unit": "GB/s" if bound == "hbm" else "TFLOP/s", "frac": round(a / p, 4),
               "traffic": traffic_for(name)}
        if bound != "hbm":
            out["dtype"] = {"fp4": "e2m1 x e2m1", "fp8": "e4m3 x e2m1", "bf16": "bf16 x bf16"}[bound]
        # single-launch figure beside the steady-state one
        out["achieved_single_median"] = round((r["bytes"] if bound == "hbm" else r["flops"])
                                              / r["ms_single_median"] / (1e6 if bound == "hbm" else 1e9), 1)
        if ceil:
            c = ceil.get({"hbm": "hbm_read_GBps", "fp4": "mfma_fp4_TFLOPs", "fp8": "mfma_fp8_TFLOPs",
                          "bf16": "mfma_bf16_TFLOPs"}[bound])
            sm = ceil.get("hbm_stream_model")
            if c and bound == "hbm" and sm:
                # the streaming model's time for the op's read and written
                # bytes: t0 + read / BW_read + written / BW_write
                w = r["bytes_written"]
                t_us = sm["t0_us"] + (r["bytes"] - w) / sm["read_GBps"] / 1e3 + w / sm["write_GBps"] / 1e3
                c = round(r["bytes"] / t_us / 1e3, 1)
            if c:
                out["ceiling"] = c
                out["frac_of_ceiling"] = round(a / c, 4)
        return out

    rooflines = {name: roof(name) for name in per_op}

    result = {
        "metric": METRIC,
        "value": per_op[HEAD]["GB/s"] if HEAD in per_op else None,
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
        "roofline": rooflines.get(HEAD),
        "secondary": None,
        "ceilings": ceil,
        "rooflines": rooflines,
        "kernels": per_op,
    }
    if "gemm_w4a4_8192" in per_op:
        r = rooflines["gemm_w4a4_8192"]
        result["secondary"] = {"metric": "W4A4 GEMM TFLOPS (8192^3, MXFP4 x MXFP4, bf16 out)",
                               "value": r["achieved"], "unit": "TFLOP/s", "frac_of_mxfp4_peak": r["frac"],
                               "frac_of_measured_mfma_ceiling": r.get("frac_of_ceiling")}
    if not args.no_metrics:
        result["metrics"] = quality_metrics(torch, mxq, keep)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------- on-box ceilings

def measure_ceilings(torch, dev, stream):
    """Ceilings measured on this machine by libmxq_ceiling.so's kernels:
    - hbm_read_GBps: the best of a small sweep (loads in flight x grid) of a
      pure streaming read of 124,854,272 bytes (the m = 1 decode GEMV's
      algorithmic bytes) per launch, rotating over copies that defeat the
      256 MB cache, burst-timed like the library's ops; hbm_read_1GiB_GBps
      the same for 1 GiB per launch;
    - hbm_write_GBps: a pure streaming write (one pass, 16-byte stores with
      the streaming hint, best of 1-8 stores per lane) of 268,435,456 bytes
      per launch, the largest output an op writes (16384 x 8192 bf16), and
      of 67,108,864 bytes;
    - hbm_stream_model: t = t0 + read bytes / BW_read + written bytes /
      BW_write, with t0 and BW_read fitted to the two read sizes and
      BW_write to the two write sizes.  An HBM op's ceiling is its bytes over
      that time for its own read and written bytes (for the m = 1 GEMV, all
      reads of the fitted size, it is hbm_read_GBps);
    - mfma_fp4_TFLOPs / mfma_bf16_TFLOPs: back-to-back 32x32 MFMAs on random
      register operands on every SIMD (8 waves per CU), with the shader clock
      read in the kernel (core-cycle counter over the constant-rate counter);
      the E4M3 x E2M1 issue ceiling is half the E2M1 one (the instruction
      takes twice the cycles).
    """
    path = os.path.join(ROOT, "mxfp4_microscaling_quantization_mxq_amd", "libmxq_ceiling.so")
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.mxqc_stream_read.argtypes = [P, I64, I, I, P, P]
    lib.mxqc_stream_write.argtypes = [P, I64, I, P]
    lib.mxqc_mfma_fp4.argtypes = [P, I64, I, P, P, P]
    lib.mxqc_mfma_bf16.argtypes = [P, I64, I, P, P, P]
    sptr = ctypes.c_void_p(stream.cuda_stream)
    out = {}

    def timed(fn, reps=5, burst=BURST):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(burst):
                fn()
            e1.record(stream)
            e1.synchronize()
            t.append(e0.elapsed_time(e1) / burst)
        return float(np.median(t))

    sink = torch.empty(65536, dtype=torch.float32, device=dev)
    for label, nbytes in (("hbm_read_GBps", 124_854_272), ("hbm_read_1GiB_GBps", 1 << 30)):
        ncp = max(2, -(-COLD_BYTES // nbytes))
        buf = torch.empty(ncp * nbytes, dtype=torch.uint8, device=dev)
        buf.fill_(0x5A)
        best = None
        for unroll in (4, 8, 16):
            for blocks in (1024, 2048, 4096, 8192):
                st = {"i": 0}

                def fn(unroll=unroll, blocks=blocks):
                    off = (st["i"] % ncp) * nbytes
                    st["i"] += 1
                    rc = lib.mxqc_stream_read(ctypes.c_void_p(buf.data_ptr() + off), nbytes, unroll, blocks,
                                              ctypes.c_void_p(sink.data_ptr()), sptr)
                    assert rc == 0, rc
                ms = timed(fn)
                gbs = nbytes / ms / 1e6
                if best is None or gbs > best[0]:
                    best = (gbs, unroll, blocks, ms)
        out[label] = round(best[0], 1)
        out[label.replace("_GBps", "_shape")] = {"loads_in_flight": best[1], "blocks": best[2],
                                                 "us": round(best[3] * 1e3, 2)}
        del buf
    wt = {}
    for nbytes in (67_108_864, 268_435_456):
        ncp = max(2, -(-COLD_BYTES // nbytes))
        buf = torch.empty(ncp * nbytes, dtype=torch.uint8, device=dev)
        best = None
        for unroll in (1, 2, 4, 8):
            st = {"i": 0}

            def fn(unroll=unroll):
                off = (st["i"] % ncp) * nbytes
                st["i"] += 1
                rc = lib.mxqc_stream_write(ctypes.c_void_p(buf.data_ptr() + off), nbytes, unroll, sptr)
                assert rc == 0, rc
            ms = timed(fn)
            if best is None or ms < best[1]:
                best = (unroll, ms)
        wt[nbytes] = best
        del buf
    out["hbm_write_GBps"] = round(268_435_456 / wt[268_435_456][1] / 1e6, 1)
    out["hbm_write_shape"] = {"bytes": 268_435_456, "stores_per_lane": wt[268_435_456][0],
                              "us": round(wt[268_435_456][1] * 1e3, 2),
                              "us_at_67108864_bytes": round(wt[67_108_864][1] * 1e3, 2)}
    # streaming model t = t0 + read bytes / BW_read + written bytes / BW_write,
    # fitted to the two read sizes (t0, BW_read) and the two write sizes
    # (BW_write); GB/s and microseconds
    r0, r1 = out["hbm_read_shape"]["us"], out["hbm_read_1GiB_shape"]["us"]
    w0, w1 = wt[67_108_864][1] * 1e3, wt[268_435_456][1] * 1e3
    if r1 > r0 and w1 > w0:  # else the rows keep the plain read ceiling
        bwr = ((1 << 30) - 124_854_272) / (r1 - r0) / 1e3
        bww = (268_435_456 - 67_108_864) / (w1 - w0) / 1e3
        out["hbm_stream_model"] = {"t0_us": round(r0 - 124_854_272 / bwr / 1e3, 2), "read_GBps": round(bwr, 1),
                                   "write_GBps": round(bww, 1)}
    src = torch.randint(0, 256, (8192,), dtype=torch.uint8, device=dev)
    wall_khz = lib.mxqc_wall_clock_khz()
    out["peak_sclk_MHz"] = lib.mxqc_peak_clock_khz() / 1e3
    for label, fnname, per_mfma in (("mfma_fp4_TFLOPs", "mxqc_mfma_fp4", 2 * 32 * 32 * 64),
                                    ("mfma_bf16_TFLOPs", "mxqc_mfma_bf16", 2 * 32 * 32 * 16)):
        blocks, iters = 1024, 2048
        clk = torch.zeros(blocks * 8 * 4, dtype=torch.int64, device=dev)
        f = getattr(lib, fnname)

        def fn():
            rc = f(ctypes.c_void_p(src.data_ptr()), iters, blocks, ctypes.c_void_p(sink.data_ptr()),
                   ctypes.c_void_p(clk.data_ptr()), sptr)
            assert rc == 0, rc
        ms = timed(fn, reps=3, burst=4)
        flops = blocks * 8 * 8 * iters * per_mfma
        out[label] = round(flops / ms / 1e9, 1)
        c = clk.view(-1, 4).cpu().numpy().astype(np.float64)
        mhz = (c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1) * wall_khz / 1e3
        out[label.replace("_TFLOPs", "_sclk_MHz")] = round(float(np.median(mhz)), 1)
    out["mfma_fp8_TFLOPs"] = round(out["mfma_fp4_TFLOPs"] / 2, 1)
    print(f"  ceilings: {json.dumps(out)}", file=sys.stderr, flush=True)
    return out


# ---------------------------------------------------------------- quality (host, untimed)

def quality_metrics(torch, mxq, keep):
    """NMSE and cosine (float64, host) of the GPU's quantized tensors and
    products: the tiny reference's W and y, and for NVFP4 and MXFP4 the
    8192x4096 W, the 4096x4096 X and the product Y = X W^T, Y against the
    product of the unquantized inputs (W4A16: only W is quantized in Y)."""
    from mxfp4_microscaling_quantization_mxq_amd.metrics import bf16_bits_to_f64, nmse_cosine
    from mxfp4_microscaling_quantization_mxq_amd import synth

    def host_bits(t):
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)

    def rnd(p):
        return [round(p[0], 6), round(p[1], 6)]

    out = {}
    if "tiny" in keep:
        w1, x1, y1, g1 = keep["tiny"]
        xf = synth.bf16_bits_to_f32(x1).astype(np.float64)
        yexact = xf @ w1.astype(np.float64).T
        out["tiny_256x512"] = {"MXFP4": {"W": rnd(nmse_cosine(w1, y1.cpu().numpy())),
                                         "Y": rnd(nmse_cosine(yexact, bf16_bits_to_f64(host_bits(g1))))}}
    if "c5" in keep:
        w5, x5, w5d, x5d, y5m, y5n = keep["c5"]
        wf = synth.bf16_bits_to_f32(w5).astype(np.float64)
        xf = synth.bf16_bits_to_f32(x5).astype(np.float64)
        yexact = xf @ wf.T
        c5 = {}
        for fmt in ("MXFP4", "NVFP4"):
            rows = {}
            for tname, tsrc, tref in (("W", w5d, wf), ("X", x5d, xf)):
                if fmt == "MXFP4":
                    q, s = mxq.quantize(tsrc)
                    deq = mxq.dequantize(q, s, torch.float32)
                else:
                    q, s, g = mxq.nv_quantize(tsrc)
                    deq = mxq.nv_dequantize(q, s, g, torch.float32)
                rows[tname] = rnd(nmse_cosine(tref, deq.cpu().numpy()))
            y = y5m if fmt == "MXFP4" else y5n
            rows["Y"] = rnd(nmse_cosine(yexact, bf16_bits_to_f64(host_bits(y))))
            c5[fmt] = rows
        out["nv_vs_mx_8192x4096x4096"] = c5
    print(f"  metrics: {json.dumps(out)}", file=sys.stderr, flush=True)
    return out


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
    the full decode GEMV (m = 1) repeated for about 8 s, the 1024 x 1024
    top-left output block of the 8192^3 W4A4 GEMM (rows 0..1023 of the
    workload's own A and B, k = 8192), and the full dynamic quantize."""
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
    a, b = synth.w4a4_operands()
    a, b = np.ascontiguousarray(a[:1024]), np.ascontiguousarray(b[:1024])
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
        "gemm_sample": f"C[0:1024, 0:1024] of the 8192^3 W4A4 GEMM: rows 0..1023 of the workload's own A and B "
                       f"(k = 8192), dequantize + double products, {t_gemm:.2f}s",
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
