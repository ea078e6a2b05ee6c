/*
 * mxq.h -- C ABI of the MI355X (gfx950) MXFP4 / NVFP4 microscaling library
 * (libmxq.so).
 *
 * Formats (the web pages these follow):
 *   - MXFP4: blocks of 32 consecutive elements along a row share one E8M0
 *     scale (a pure power of two, code c means 2^(c-127)); each element is an
 *     E2M1 code (1 sign, 2 exponent, 1 mantissa bit; magnitudes
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}).  4.25 bits per element.
 *     ["4.5 FP8 and NVFP4/MXFP4" (infra-guide), sec. 3.1, 3.3 and the
 *     sec. 4.1 table; MXFP4 explainer (mingyuyang.com AI daily,
 *     2026-08-05), sec. 3.]
 *   - NVFP4: blocks of 16 share an E4M3 block scale, and the whole tensor
 *     shares one FP32 scale: x_hat = s_tensor * s_block * q.  4.5 bits per
 *     element plus the tensor scale.  [infra-guide sec. 4.1; TransFP4 page
 *     "Portable FP4 quantization for heterogeneous accelerators",
 *     sec. 1.1 eq. (1).]
 *
 * Quantization rules (the pages give the idea -- the block's largest
 * magnitude is mapped onto the top of the E2M1 range by the shared scale,
 * with nearest rounding -- and this library fixes the details):
 *   MXFP4 scale exponent e = floor(log2(amax_block)) - 2, clamped to
 *   [-127, 127] (an all-zero block gets code 0); element code =
 *   E2M1 round-to-nearest-even of x * 2^-e, saturated to +-6, sign kept
 *   (so -0 and tiny negatives give code 0x8).
 *   NVFP4 tensor scale s_t = fl32(amax_tensor / 2688) (2688 = 6 * 448; 1 for
 *   an all-zero tensor), stored as the DEQUANTIZATION multiplier; block
 *   scale s_b = E4M3_rne_saturating(fl32(amax_block / fl32(6 * s_t)));
 *   element code = E2M1_rne(fl32(x / fl32(s_t * s_b))), or signed zero when
 *   s_b encodes to 0.
 *
 * Layout: every matrix is row-major with no padding ([rows][k], k
 * contiguous); quantization blocks run along k.  Packed codes q[rows][k/2]
 * hold element 2j in the LOW nibble of byte j and element 2j+1 in the high
 * nibble.  Scales are one byte per block: s[rows][k/32] (E8M0) or
 * s[rows][k/16] (E4M3).  Products use the linear-layer ("NT") form
 *   Y[i][j] = sum_t X[i][t] * W[j][t].
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers on the current HIP device, except
 *     mxq_status_string's result (a static host string).
 *   - The caller owns every buffer.  The library never allocates, frees,
 *     synchronizes, or keeps a pointer after the call returns.  Outputs must
 *     not alias inputs.  Work is enqueued on `stream` (0 = default stream)
 *     and the call returns without waiting for it.
 *   - Validation happens before anything is launched; on any error nothing
 *     is written.  Any size (rows, k, m or n) below 1 ->
 *     MXQ_ERROR_INVALID_VALUE: an empty problem is rejected, not a no-op.
 *     k not a multiple of the block size -> MXQ_ERROR_INVALID_VALUE.  A NULL
 *     pointer -> MXQ_ERROR_INVALID_VALUE.  A base pointer
 *     that is not 16-byte aligned (4-byte for the scalar NVFP4 tensor scale)
 *     -> MXQ_ERROR_MISALIGNED.  No HIP device, or a device that is not
 *     gfx950 -> MXQ_ERROR_NOT_SUPPORTED.  A failed launch ->
 *     MXQ_ERROR_LAUNCH_FAILURE.  Faults inside a kernel are asynchronous and
 *     surface at the caller's next synchronization.
 * *   - Non-finite inputs (NaN, Inf) are outside the contract.  Products whose
 *     exact value, or whose dequantized operands, leave the fp32 range
 *     (scale codes above 250 or below about 16) are outside the contract.
 *   - Results are deterministic: the same call gives bitwise identical
 *     output on every run.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_API __attribute__((visibility("default")))

/* The *_MAX_ENUM members are never returned or accepted as valid; they give
 * both enums the whole non-negative int range, so any int a caller passes
 * (e.g. an unknown status code to mxq_status_string, or a bad dtype that
 * validation rejects) is a value of the type. */
typedef enum {
    MXQ_SUCCESS = 0,
    MXQ_ERROR_INVALID_VALUE = 1,
    MXQ_ERROR_MISALIGNED = 2,
    MXQ_ERROR_NOT_SUPPORTED = 3,
    MXQ_ERROR_LAUNCH_FAILURE = 4,
    MXQ_STATUS_MAX_ENUM = 0x7FFFFFFF
} mxq_status;

/* Element type of an unquantized operand: fp32, or bf16 (bfloat16). */
typedef enum { MXQ_F32 = 0, MXQ_BF16 = 1, MXQ_DTYPE_MAX_ENUM = 0x7FFFFFFF } mxq_dtype;

/* Static, NUL-terminated description of a status code (host memory). */
MXQ_API const char *mxq_status_string(mxq_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
MXQ_API int mxq_version(void);

/*
 * MXFP4 quantize.  x[rows][k] of type xdt (MXQ_F32 or MXQ_BF16) ->
 * q[rows][k/2] packed E2M1 codes and s[rows][k/32] E8M0 scale codes.
 * Online (calibration-free) quantization from 16- or 32-bit values, as in
 * load-time conversion of a BF16 checkpoint [infra-guide sec. 4.2].
 * k % 32 == 0 is required (32-aligned K is the kernel contract, TransFP4
 * page sec. 2.2 Table 3).
 */
MXQ_API mxq_status mxq_quantize(const void *x, mxq_dtype xdt, int64_t rows, int64_t k,
                        uint8_t *q, uint8_t *s, hipStream_t stream);

/*
 * Rotated MXFP4 quantize: the MXFP4 codes and scales (as mxq_quantize) of
 * y = x rotated block by block along k with H_hk, the Sylvester-ordered
 * Hadamard matrix divided by sqrt(hk) (orthonormal and symmetric, so the
 * rotation is undone by applying it again, and Y = X W^T equals the product
 * of the rotated X and W).  hk is 16, 32, 64 or 128; k % 32 == 0 and
 * k % hk == 0.  The rotation is computed in fp32 in a fixed order: butterfly
 * stages h = 1, 2, ..., hk/2, each pair (i, i + h) -> (u + v, u - v), then
 * a multiply by the fp32 nearest 1/sqrt(hk); the codes are decided on those
 * fp32 values.  x[rows][k] (xdt), q[rows][k/2], s[rows][k/32].
 * [TransFP4 page sec. 2.3 eq. (2): an orthogonal H_j per block keeps the
 * 2-norm; "FP4 quantization analysis" page sec. 3.2.3: block-diagonal
 * Hadamard H_k, k in {16, 32, 64, 128}, computed online for activations.]
 * Errors: INVALID_VALUE for any other hk or a k not a multiple of 32 and
 * hk, as well as the cases of mxq_quantize.
 */
MXQ_API mxq_status mxq_quantize_hadamard(const void *x, mxq_dtype xdt, int64_t rows,
                                 int64_t k, int hk, uint8_t *q, uint8_t *s,
                                 hipStream_t stream);

/*
 * MXFP8 quantize.  x[rows][k] (xdt) -> q[rows][k] E4M3 codes (one byte per
 * element) and s[rows][k/32] E8M0 scale codes.  Block exponent e =
 * floor(log2 amax) - 8, clamped to [-127, 127] (448 = 1.75 * 2^8 is E4M3's
 * largest value, so the block's largest magnitude scales into [256, 512));
 * elements E4M3(x * 2^-e), round to nearest even, saturating at 448, sign
 * of zero kept.  k % 32 == 0.  [infra-guide "4.5 FP8 and NVFP4/MXFP4" sec.
 * 4.2: the mxfp8 scheme, FP8 values with an E8M0 scale per 1x32; sec. 1.2:
 * E4M3 range and NaN-only special value.]  Errors as mxq_quantize.
 */
MXQ_API mxq_status mxq_quantize_fp8(const void *x, mxq_dtype xdt, int64_t rows, int64_t k,
                            uint8_t *q, uint8_t *s, hipStream_t stream);

/*
 * MXFP4 dequantize.  (q[rows][k/2], s[rows][k/32]) -> y[rows][k] of type ydt:
 * y = E2M1(code) * 2^(s - 127), exact in fp32 and bf16 for scale codes
 * 1..250 [TransFP4 page eq. (1) with s_g = 1].  Scale code 255 (NaN in E8M0)
 * gives NaN.
 */
MXQ_API mxq_status mxq_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows,
                          int64_t k, void *y, mxq_dtype ydt,
                          hipStream_t stream);

/*
 * W4A16 product with an MXFP4 weight: y[m][n] = sum_k x[m][k] * W_hat[n][k],
 * where W = (wq[n][k/2], ws[n][k/32]) is dequantized in registers (never
 * written out in 16 bits), x[m][k] is bf16, accumulation is fp32, and y is
 * written as ydt (MXQ_F32 or MXQ_BF16, round to nearest even).  Weight-only
 * 4-bit with 16-bit multiplies saves bandwidth, not arithmetic
 * [infra-guide sec. 4.2 and 5].  Any m >= 1.  Memory-bound decode kernels
 * up to m = 127; for n >= 14336 and k % 512 == 0 a weight-streaming ring of
 * up to 64 activation rows, with m = 65..128 as two launches of it.  Larger
 * m takes a bf16-MFMA GEMM tile (for k < 2^23; longer rows stay on the
 * decode kernels).  k % 32 == 0.
 */
MXQ_API mxq_status mxq_gemv_w4a16(const uint8_t *wq, const uint8_t *ws, int64_t n,
                          int64_t k, const void *x, int64_t m, void *y,
                          mxq_dtype ydt, hipStream_t stream);

/*
 * W4A4 product of two MXFP4 operands on the gfx950 block-scaled MFMA:
 * c[m][n] = sum_k A_hat[m][k] * B_hat[n][k], A = (aq[m][k/2], as[m][k/32]),
 * B = (bq[n][k/2], bs[n][k/32]); fp32 accumulation; c written as cdt.
 * Native FP4 matrix math needs both operands quantized [infra-guide sec. 5];
 * CDNA 4 provides exponent-block-scaled matrix instructions [TransFP4 page
 * sec. 5.1].  k % 32 == 0.
 */
MXQ_API mxq_status mxq_gemm_w4a4(const uint8_t *aq, const uint8_t *as,
                         const uint8_t *bq, const uint8_t *bs, int64_t m,
                         int64_t n, int64_t k, void *c, mxq_dtype cdt,
                         hipStream_t stream);

/*
 * W4A8 product: c[m][n] = sum_k A_hat[m][k] * B_hat[n][k] with MXFP8
 * activations A = (aq8[m][k] E4M3, as[m][k/32]) and MXFP4 weights
 * B = (bq[n][k/2], bs[n][k/32]), on the block-scaled MFMA that takes an
 * E4M3 and an E2M1 operand; fp32 accumulation; c written as cdt.  k % 32 ==
 * 0.  [Kimi K3 release format: MXFP4 weights with MXFP8 activations, "Low-
 * precision inference and MXFP4 quantization" page; mxfp8 scheme, infra-
 * guide sec. 4.2.]  Errors as mxq_gemm_w4a4.
 * Accuracy: the instruction adds the products of each group of 8
 * consecutive k aligned to the group's largest exponent E_g (the two codes'
 * exponents summed) and truncated toward zero at 2^(E_g - 13), before the
 * block scales and the fp32 accumulation (measured on gfx950), so a group
 * can lose up to about 8 * 2^(E_g - 13) times its two block scales; with
 * at most one nonzero activation per group the result is fp32-accurate.
 */
MXQ_API mxq_status mxq_gemm_w4a8(const uint8_t *aq8, const uint8_t *as,
                         const uint8_t *bq, const uint8_t *bs, int64_t m,
                         int64_t n, int64_t k, void *c, mxq_dtype cdt,
                         hipStream_t stream);

/*
 * W4A4 product with MXFP4 output: c = bf16(A_hat B_hat^T) computed as in
 * mxq_gemm_w4a4 with bf16 output, then quantized to MXFP4 along n in the
 * kernel's epilogue, so the 16-bit product never reaches memory.  The codes
 * cq[m][n/2] and E8M0 scales cs[m][n/32] are bit-identical to mxq_quantize
 * of the bf16 product (the same quantizer runs on the same bf16 values).
 * n % 32 == 0, k % 32 == 0.
 * [TransFP4 page sec. 2.5: no 16-bit copy is materialized; "FP4
 * quantization analysis" page, QuTLASS kernel section: custom epilogues
 * fuse the quantization of the output.]
 */
MXQ_API mxq_status mxq_gemm_w4a4_quant(const uint8_t *aq, const uint8_t *as,
                               const uint8_t *bq, const uint8_t *bs, int64_t m,
                               int64_t n, int64_t k, uint8_t *cq, uint8_t *cs,
                               hipStream_t stream);

/*
 * W4A4 product from bf16 activations quantized inside the kernel:
 * c[m][n] = sum_k MXFP4(x)[m][k] * B_hat[n][k], where MXFP4(x) is exactly
 * what mxq_quantize writes for x (the same quantizer runs on the same
 * values), so c is bit-identical to mxq_quantize followed by mxq_gemm_w4a4.
 * The activation codes never reach memory.  [TransFP4 page sec. 2.5: format
 * conversion belongs in the GEMM's load stage, not in a separate
 * intermediate tensor; "FP4 quantization analysis" page, QuTLASS kernel
 * section: quantization fused into the GEMM kernels.]
 * x bf16 [m][k]; B = (bq[n][k/2], bs[n][k/32]); fp32 accumulation; c
 * written as cdt.  For decode-sized batches only: every block of 112
 * weight rows quantizes the bf16 activation tile again, which pays while the
 * weight stream dominates.  1 <= m <= 16, k % 512 == 0, k <= 2^24, else
 * MXQ_ERROR_INVALID_VALUE (larger batches: mxq_quantize once, then
 * mxq_gemm_w4a4, which is faster there).  Errors otherwise as
 * mxq_gemm_w4a4.
 */
MXQ_API mxq_status mxq_gemm_w4a4_dynamic(const void *x, const uint8_t *bq,
                                 const uint8_t *bs, int64_t m, int64_t n,
                                 int64_t k, void *c, mxq_dtype cdt,
                                 hipStream_t stream);

/*
 * W4A8 product from bf16 activations quantized to MXFP8 inside the kernel:
 * c[m][n] = sum_k MXFP8(x)[m][k] * B_hat[n][k], where MXFP8(x) is exactly
 * what mxq_quantize_fp8 writes for x, so c is bit-identical to
 * mxq_quantize_fp8 followed by mxq_gemm_w4a8 (whose accuracy note applies).
 * [MXFP8 activations with a dynamic per-token-block quantization: infra-
 * guide sec. 4.2 (mxfp8); TransFP4 page sec. 2.5: conversion in the GEMM's
 * load stage.]  x bf16 [m][k]; B = (bq[n][k/2], bs[n][k/32]); c written as
 * cdt.  For decode-sized batches, as mxq_gemm_w4a4_dynamic: 1 <= m <= 16,
 * k % 512 == 0, k <= 2^24, else MXQ_ERROR_INVALID_VALUE (larger batches:
 * mxq_quantize_fp8 once, then mxq_gemm_w4a8, which is faster there).
 * Errors otherwise as mxq_gemm_w4a4.
 */
MXQ_API mxq_status mxq_gemm_w4a8_dynamic(const void *x, const uint8_t *bq,
                                 const uint8_t *bs, int64_t m, int64_t n,
                                 int64_t k, void *c, mxq_dtype cdt,
                                 hipStream_t stream);

/*
 * NVFP4 quantize.  x[rows][k] (xdt) -> q[rows][k/2] packed E2M1 codes,
 * s[rows][k/16] E4M3 block-scale codes, and the fp32 tensor scale *gscale
 * (a single float in device memory, the dequantization multiplier).
 * compute_gscale != 0: the library computes s_t from the tensor's amax and
 * writes it to *gscale (the caller's value is overwritten).  compute_gscale
 * == 0: *gscale is read as given (a static, pre-computed scale; it must be
 * finite and > 0).  k % 16 == 0.  [infra-guide sec. 2 and 4.1.]
 */
MXQ_API mxq_status nvq_quantize(const void *x, mxq_dtype xdt, int64_t rows, int64_t k,
                        float *gscale, int compute_gscale, uint8_t *q,
                        uint8_t *s, hipStream_t stream);

/*
 * NVFP4 dequantize: y = (*gscale) * E4M3(s) * E2M1(q), written as ydt.
 * E4M3(s) * E2M1(q) is exact; the product with the fp32 tensor scale is
 * rounded ONCE, to nearest even, to ydt (fp32 or bf16).  k % 16 == 0.
 */
MXQ_API mxq_status nvq_dequantize(const uint8_t *q, const uint8_t *s,
                          const float *gscale, int64_t rows, int64_t k,
                          void *y, mxq_dtype ydt, hipStream_t stream);

/*
 * W4A16 product with an NVFP4 weight, software two-level dequantization:
 * y[m][n] = s_t * sum_k x[m][k] * (E4M3(ws[n][k/16]) * E2M1(wq[n][k])),
 * bf16 MFMA with fp32 accumulation and the tensor scale *wgscale applied
 * once in the epilogue.  The block scale is applied either to the codes
 * (s_b * q formed exactly in bf16 in registers) or, for up to 8 activation
 * rows on weights of at least 14336 rows, to each 16-k block's fp32 sum of
 * the exact unscaled products (one fp32 multiply-add per block and output);
 * either way the result is held to the same bound against the exact sum.
 * x[m][k] bf16; y written as ydt.  k % 16 == 0.
 * [infra-guide sec. 4.1: x_hat = s_tensor * s_block * q; TransFP4 page
 * sec. 2.5: scales are decoded at matrix load, no 16-bit copy of W.]
 */
MXQ_API mxq_status nvq_gemm(const uint8_t *wq, const uint8_t *ws, const float *wgscale,
                    int64_t n, int64_t k, const void *x, int64_t m, void *y,
                    mxq_dtype ydt, hipStream_t stream);

/*
 * TransFP4 quantize [TransFP4 page sec. 2.3 eq. (3): x_hat = H^T Q_f(Hx -
 * P_r Hx) + H^T P_r Hx; sec. 3.1: 32-point Hadamard, at most one residual
 * per 32 values, per-block choice between the NVFP4 and the INT4 candidate
 * by block error; sec. 2.2 Table 3: a 16-bit residual lane and a format
 * tag].  Per 32-element block of x[rows][k] (xdt) along k:
 *   - y = H_32 x in fp32 (the order of mxq_quantize_hadamard);
 *   - the residual: the position of the largest |y_i| (first on ties) and
 *     that value rounded to bf16; the position is set to +0;
 *   - candidates under one E4M3 scale per 16 and the fp32 tensor scale s_t:
 *     E2M1 codes (16-block amax mapped to 6) or INT4 codes (sign and
 *     magnitude 0..7, nearest even, amax mapped to 7), each with the fp32
 *     order t = fl(Q s_t), s_b = E4M3(fl(amax / t)), d = fl(s_t s_b),
 *     c = code(fl(y / d));
 *   - INT4 is kept only if its error SSE = sum fl(e_i^2), e_i =
 *     fl(y_i - fl(c_i d)), summed in fp32 as four sequential runs of 8
 *     followed by (P0 + P1) + (P2 + P3), is strictly smaller.
 * Outputs: q[rows][k/2] codes (element 2j in the low nibble), s[rows][k/16]
 * E4M3 codes, meta[rows][k/32] (bit 7 = INT4, bits 0-4 = residual
 * position), res[rows][k/32] bf16 residual bits, and *gscale = s_t.
 * compute_gscale != 0: s_t = fl(amax' / 2688) over the residual-free
 * rotated tensor (1 if it is all zero) is computed and written (q serves as
 * scratch for the partial maxima before it receives the codes); == 0:
 * *gscale is read (finite, > 0).  k % 32 == 0; every array 16-byte aligned,
 * gscale 4-byte aligned.  Errors as nvq_quantize.
 */
MXQ_API mxq_status mxq_transfp4_quantize(const void *x, mxq_dtype xdt, int64_t rows, int64_t k,
                                 float *gscale, int compute_gscale, uint8_t *q, uint8_t *s,
                                 uint8_t *meta, uint16_t *res, hipStream_t stream);

/*
 * TransFP4 dequantize: y_hat_i = fl(c_i * fl(s_t * E4M3(s_h))) with the
 * codebook the block's tag selects, plus the bf16 residual at its
 * position, then x_hat = H_32 y_hat (H is symmetric and orthonormal, so
 * H^T = H) in the same fp32 butterfly order; written as ydt (bf16: the fp32
 * result rounded to nearest even).  Layout as mxq_transfp4_quantize.
 */
MXQ_API mxq_status mxq_transfp4_dequantize(const uint8_t *q, const uint8_t *s,
                                   const uint8_t *meta, const uint16_t *res,
                                   const float *gscale, int64_t rows, int64_t k, void *y,
                                   mxq_dtype ydt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
