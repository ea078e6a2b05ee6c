/*
 * mxq_oracle.c -- plain, slow, obviously-correct CPU oracle for OCP MXFP4
 * and NVFP4 microscaling.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path (the HIP library and
 * its Python binding) may include, link, load or call this file.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no header, table, helper or constant with the GPU sources.
 *
 * Sources (the web pages the method is described on):
 *   [EXPLAINER]  "Low-precision inference and MXFP4 quantization"
 *                (mingyuyang.com AI daily, 2026-08-05), sec. 3 "Core idea:
 *                block scaling makes 4 bits usable".
 *   [TRANSFP4]   "Portable FP4 quantization for heterogeneous accelerators"
 *                (elexvx.com research), sec. 1.1 eq. (1), sec. 3.1, sec. 3.2.
 *   [GUIDE]      "4.5 FP8 and NVFP4/MXFP4" (infra-guide, inference
 *                optimization ch. 4), sec. 1.1, 1.2, 2, 3.1, 3.3, 4.1.
 *   [GPTOSS]     gpt-oss MXFP4 repost (juejin.cn post 7539732578421833769),
 *                section "MXFP4" with the four-value worked example.
 *   [ANALYSIS]   "FP4 quantization analysis: MXFP4 and NVFP4 compared, in
 *                practice" (jsqmd.com news), sec. 3.2.3 "fused online
 *                rotation" (block-diagonal Hadamard H_k, k in 16..128).
 *
 * Precision discipline: every MXFP4 decision is exact (power-of-two scaling
 * of a float in double, then nearest-value search in double).  NVFP4 works
 * in IEEE fp32 because its tensor scale is an FP32 number [GUIDE sec. 4.1];
 * build with -ffp-contract=off and without fast-math so each fp32 operation
 * rounds once, to nearest even.  Products accumulate in double.
 *
 * Readings the pages leave open (each one is listed in the design notes):
 *   - E2M1 ties: round-to-nearest-even by default; a ties-away mode exists
 *     only to reproduce the worked example as printed [GPTOSS].
 *   - E8M0 exponent: e = floor(log2 amax) - 2, clamped to [-127, 127];
 *     an all-zero block takes e = -127 (scale code 0).
 *   - Nibble order: element 2j in the low nibble of byte j.
 *   - NVFP4 tensor scale: s_t = amax_t / (6 * 448) in fp32, stored as the
 *     dequantization multiplier; s_t = 1 for an all-zero tensor.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1

/* ------------------------------------------------------------------ */
/* Element formats                                                     */
/* ------------------------------------------------------------------ */

/* E2M1 value of a 4-bit code [GUIDE sec. 3.1]: one sign bit, two exponent
 * bits, one mantissa bit (S EE M from the most significant bit).  With
 * exponent bias 1, E = 0 is subnormal with step 0.5, and the largest value
 * is 2^2 * 1.5 = 6, as the guide states. */
double or_e2m1_decode(uint8_t code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag;
    if (e == 0)
        mag = 0.5 * m;
    else
        mag = ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E2M1 encode: the representable magnitude nearest to |v|; magnitudes at or
 * above the largest value (6) saturate to 6.
 * An exact tie between two neighbours goes to the code whose mantissa bit is
 * 0 (round half to even), or, in ties_away mode, to the larger magnitude.
 * The sign bit copies the sign of v, so -0 and small negatives give 0x8. */
uint8_t or_e2m1_encode(double v, int ties_away)
{
    double a = fabs(v);
    int best = 0;
    double bestd = INFINITY;
    if (a >= 6.0) /* saturate: explicit, so huge |v| never ties in rounding */
        return (uint8_t)(7 | (signbit(v) ? 8 : 0));
    for (int c = 0; c < 8; c++) {
        double d = fabs(a - or_e2m1_decode((uint8_t)c));
        if (d < bestd) {
            best = c;
            bestd = d;
        } else if (d == bestd) {
            /* tie between best (smaller magnitude) and c (larger) */
            if (ties_away)
                best = c;
            else if ((c & 1) == 0)
                best = c;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 8 : 0));
}

/* E4M3 value of an 8-bit code [GUIDE sec. 1.1-1.2]: S EEEE MMM, bias 7
 * (bits 00111000 read as 1.0), subnormals for E = 0, no infinities, and the
 * single all-ones pattern S 1111 111 is NaN, so the largest finite value is
 * 2^8 * 1.75 = 448. */
double or_e4m3_decode(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp(m / 8.0, -6);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E4M3 encode of a non-negative fp32 value: nearest finite E4M3 value,
 * ties to the code with mantissa LSB 0, saturating at 448 (a real type cast,
 * not rounding to an integer grid [GUIDE sec. 1.2 key point]).  Negative
 * inputs encode their magnitude with the sign bit set. */
uint8_t or_e4m3_encode(float r)
{
    double a = fabs((double)r);
    int best = 0;
    double bestd = INFINITY;
    if (a >= 448.0) /* saturate at the largest finite value, never NaN */
        return (uint8_t)(0x7E | (signbit(r) ? 0x80 : 0));
    for (int c = 0; c < 0x7F; c++) { /* 0x7F is NaN */
        double d = fabs(a - or_e4m3_decode((uint8_t)c));
        if (d < bestd) {
            best = c;
            bestd = d;
        } else if (d == bestd && (c & 1) == 0) {
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(r) ? 0x80 : 0));
}

/* ------------------------------------------------------------------ */
/* Input widening (definitions of the storage types)                   */
/* ------------------------------------------------------------------ */

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float load_elem(const void *x, int dtype, int64_t i)
{
    if (dtype == OR_BF16)
        return bf16_to_f32(((const uint16_t *)x)[i]);
    return ((const float *)x)[i];
}

void or_to_f64(const void *x, int dtype, int64_t n, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        y[i] = (double)load_elem(x, dtype, i);
}

/* ------------------------------------------------------------------ */
/* MXFP4                                                               */
/* ------------------------------------------------------------------ */

/* Shared block exponent.  The block's largest magnitude is mapped near the
 * largest E2M1 value by a power-of-two scale [EXPLAINER sec. 3; TRANSFP4
 * sec. 1.1: an E8M0 scale is a pure exponent].  Rule: e = floor(log2 amax)
 * - 2, clamped to the E8M0 range [-127, 127]; amax = 0 gives -127. */
int or_e8m0_exponent(double amax)
{
    if (amax == 0.0)
        return -127;
    int ex;
    frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex-1 */
    int e = (ex - 1) - 2;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* E8M0 scale value: 2^(code - 127); code 255 is NaN. */
double or_e8m0_decode(uint8_t code)
{
    if (code == 255)
        return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* Quantize rows x[rows][k] along k in blocks of 32 [GUIDE sec. 4.1 table:
 * 32 E2M1 elements share one E8M0 scale].  Eq. (1) of [TRANSFP4] with
 * s_g = 1: q_i = Q(x_i / s_b).  Outputs: q[rows][k/2] packed nibbles (element
 * 2j low), s[rows][k/32] E8M0 codes.  k must be a multiple of 32. */
void or_mx_quantize(const void *x, int dtype, int64_t rows, int64_t k,
                    uint8_t *q, uint8_t *s, int ties_away)
{
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            int64_t base = r * k + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; i++) {
                double a = fabs((double)load_elem(x, dtype, base + i));
                if (a > amax)
                    amax = a;
            }
            int e = or_e8m0_exponent(amax);
            s[r * nb + b] = (uint8_t)(e + 127);
            uint8_t codes[32];
            for (int i = 0; i < 32; i++) {
                double v = ldexp((double)load_elem(x, dtype, base + i), -e);
                codes[i] = or_e2m1_encode(v, ties_away);
            }
            for (int j = 0; j < 16; j++)
                q[r * (k / 2) + b * 16 + j] =
                    (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
    }
}

/* Dequantize: x_hat = E2M1(c) * 2^(s - 127), exact in double. */
void or_mx_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows,
                      int64_t k, double *y)
{
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t i = 0; i < k; i++) {
            uint8_t byte = q[r * (k / 2) + i / 2];
            uint8_t c = (i & 1) ? (byte >> 4) : (byte & 15);
            y[r * k + i] =
                or_e2m1_decode(c) * or_e8m0_decode(s[r * nb + i / 32]);
        }
    }
}

/* ------------------------------------------------------------------ */
/* MXFP8 (E4M3 elements, one E8M0 scale per 32)                        */
/* ------------------------------------------------------------------ */

/* MXFP8: FP8 values with one E8M0 scale per 1x32 block [GUIDE sec. 4.2
 * table, the mxfp8 scheme]; used for activations next to MXFP4 weights
 * [EXPLAINER, Kimi K3 release format].  The element is E4M3 (max 448 =
 * 2^8 * 1.75, NaN only [GUIDE sec. 1.2]).  Block exponent by the same rule
 * as MXFP4 with the element's top exponent: e = floor(log2 amax) - 8,
 * clamped to [-127, 127] (amax = 0: -127), so the block's largest magnitude
 * scales into [256, 512) and anything above 448 saturates; elements are
 * E4M3(x * 2^-e) rounded to nearest even. */
int or_e8m0_exponent_e4m3(double amax)
{
    if (amax == 0.0)
        return -127;
    int ex;
    frexp(amax, &ex); /* floor(log2 amax) = ex - 1 */
    int e = (ex - 1) - 8;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* x[rows][k] -> q[rows][k] E4M3 codes, s[rows][k/32] E8M0 codes. */
void or_mx8_quantize(const void *x, int dtype, int64_t rows, int64_t k,
                     uint8_t *q, uint8_t *s)
{
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            int64_t base = r * k + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; i++) {
                double a = fabs((double)load_elem(x, dtype, base + i));
                if (a > amax)
                    amax = a;
            }
            int e = or_e8m0_exponent_e4m3(amax);
            s[r * nb + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; i++) {
                /* x * 2^-e is exact in fp32 (a power-of-two scaling of an
                 * fp32/bf16 value that stays below 512 in magnitude) */
                float v = (float)ldexp((double)load_elem(x, dtype, base + i), -e);
                q[base + i] = or_e4m3_encode(v);
            }
        }
    }
}

/* Dequantize: x_hat = E4M3(c) * 2^(s - 127), exact in double. */
void or_mx8_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows,
                       int64_t k, double *y)
{
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t i = 0; i < k; i++)
            y[r * k + i] = or_e4m3_decode(q[r * k + i]) *
                           or_e8m0_decode(s[r * nb + i / 32]);
}

/* ------------------------------------------------------------------ */
/* NVFP4                                                               */
/* ------------------------------------------------------------------ */

/* Tensor scale [GUIDE sec. 2 and 4.1]: by the max rule s = max|x| / F_max,
 * stored as the dequantization multiplier.  For the two-level format the
 * largest magnitude must land on E2M1's 6 with the block scale at E4M3's
 * 448, so F_max = 6 * 448 = 2688.  An all-zero tensor takes s_t = 1. */
float or_nv_tensor_scale(float amax)
{
    if (amax == 0.0f)
        return 1.0f;
    return amax / 2688.0f;
}

/* Quantize rows x[rows][k] along k in blocks of 16 [GUIDE sec. 4.1]:
 * x_hat = s_tensor * s_block * q.  fp32 order of operations:
 *   t   = fl(6 * s_t)
 *   s_b = E4M3(fl(amax_b / t))
 *   d   = fl(s_t * E4M3value(s_b));  v_i = fl(x_i / d);  q_i = E2M1(v_i)
 * and a block whose scale encodes to zero stores signed-zero codes.  With
 * compute_gscale != 0 the tensor scale is computed and written to *gscale,
 * otherwise *gscale is read.  Outputs q[rows][k/2], s[rows][k/16]. */
void or_nv_quantize(const void *x, int dtype, int64_t rows, int64_t k,
                    float *gscale, int compute_gscale, uint8_t *q, uint8_t *s)
{
    int64_t nb = k / 16;
    if (compute_gscale) {
        float amax = 0.0f;
        for (int64_t i = 0; i < rows * k; i++) {
            float a = fabsf(load_elem(x, dtype, i));
            if (a > amax)
                amax = a;
        }
        *gscale = or_nv_tensor_scale(amax);
    }
    const float st = *gscale;
    const float t = 6.0f * st;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            int64_t base = r * k + b * 16;
            float amax = 0.0f;
            for (int i = 0; i < 16; i++) {
                float a = fabsf(load_elem(x, dtype, base + i));
                if (a > amax)
                    amax = a;
            }
            float ratio = amax / t;
            uint8_t sb = or_e4m3_encode(ratio);
            s[r * nb + b] = sb;
            float sbv = (float)or_e4m3_decode(sb);
            uint8_t codes[16];
            for (int i = 0; i < 16; i++) {
                float xi = load_elem(x, dtype, base + i);
                if (sbv == 0.0f) {
                    codes[i] = (uint8_t)(signbit(xi) ? 8 : 0);
                } else {
                    float d = st * sbv;
                    float v = xi / d;
                    codes[i] = or_e2m1_encode((double)v, 0);
                }
            }
            for (int j = 0; j < 8; j++)
                q[r * (k / 2) + b * 8 + j] =
                    (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
    }
}

/* Dequantize: x_hat = s_t * E4M3(s_b) * E2M1(c), exact in double. */
void or_nv_dequantize(const uint8_t *q, const uint8_t *s, float gscale,
                      int64_t rows, int64_t k, double *y)
{
    int64_t nb = k / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t i = 0; i < k; i++) {
            uint8_t byte = q[r * (k / 2) + i / 2];
            uint8_t c = (i & 1) ? (byte >> 4) : (byte & 15);
            y[r * k + i] = (double)gscale *
                           or_e4m3_decode(s[r * nb + i / 16]) *
                           or_e2m1_decode(c);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Block Hadamard rotation ahead of quantization                       */
/* ------------------------------------------------------------------ */

/* An orthogonal H per block, y_j = H_j x_j, which keeps the 2-norm, so the
 * quantization error can be judged in the rotated domain [TRANSFP4 sec. 2.3
 * eq. (2)]; the activation side computes X H_k online with a butterfly
 * network, k in {16, 32, 64, 128} [ANALYSIS sec. 3.2.3].
 *
 * H_hk here is the Sylvester-ordered Hadamard matrix divided by sqrt(hk)
 * (orthonormal, symmetric): H[i][j] = (-1)^popcount(i & j) / sqrt(hk).  In
 * fp32 the rotation is not exact, so its order of operations is part of the
 * definition (the codes are decided on the rotated fp32 values): the fast
 * transform over h = 1, 2, 4, ..., hk/2, every pair (i, i + h) with
 * (i & h) == 0 replaced by (u + v, u - v), each sum rounded to fp32, then
 * every element multiplied by the fp32 number nearest 1/sqrt(hk). */
static float hadamard_norm_f32(int hk)
{
    return (float)(1.0 / sqrt((double)hk));
}

static void fwht_block_f32(float *v, int hk)
{
    for (int h = 1; h < hk; h *= 2)
        for (int i = 0; i < hk; i++)
            if ((i & h) == 0) {
                float u = v[i], w = v[i + h];
                v[i] = u + w;
                v[i + h] = u - w;
            }
    const float c = hadamard_norm_f32(hk);
    for (int i = 0; i < hk; i++)
        v[i] = v[i] * c;
}

float or_hadamard_norm(int hk) { return hadamard_norm_f32(hk); }

/* y[rows][k] (fp32) = x rotated block by block along k with H_hk; k must be
 * a multiple of hk. */
void or_hadamard_rotate(const void *x, int dtype, int64_t rows, int64_t k,
                        int hk, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < k / hk; b++) {
            float *v = y + r * k + b * hk;
            for (int i = 0; i < hk; i++)
                v[i] = load_elem(x, dtype, r * k + b * hk + i);
            fwht_block_f32(v, hk);
        }
    }
}

/* ------------------------------------------------------------------ */
/* TransFP4 blocks: rotation + sparse residual + FP4/INT4 choice        */
/* ------------------------------------------------------------------ */

/* [TRANSFP4 sec. 2.3 eq. (3)]: x_hat_j = H^T Q_f(H x_j - P_r H x_j)
 * + H^T P_r H x_j, where P_r keeps r positions of the rotated block in a
 * separate higher-precision residual stream; [TRANSFP4 sec. 3.1]: a 32-point
 * Hadamard, at most one residual per 32 values, and per block the NVFP4 or
 * the INT4 candidate, whichever has the smaller block error; [TRANSFP4 sec.
 * 2.2 Table 3]: the residual lane keeps one 16-bit value per 32; the format
 * tag selects the element codebook (E2M1 or INT4).
 *
 * Readings (the page leaves them open; listed in the design notes):
 *   - rotation: H_32 exactly as or_hadamard_rotate (fp32 butterfly order);
 *   - residual: the position of the largest |y_i| (lowest index on ties),
 *     value rounded to bf16 (nearest even); that position is set to +0 in
 *     the block the codebook quantizes;
 *   - both candidates use the NVFP4 two-level scale: one E4M3 scale per 16
 *     under the fp32 tensor scale s_t = amax'/2688 (amax' over the rotated,
 *     residual-free tensor); the NVFP4 candidate maps the 16-block amax to
 *     E2M1's 6, the INT4 candidate to 7, with the same fp32 order as
 *     or_nv_quantize (t = fl(Q s_t), s_b = E4M3(fl(amax/t)),
 *     d = fl(s_t E4M3(s_b)), v = fl(y/d));
 *   - INT4: sign and magnitude, magnitudes 0..7, round half to even,
 *     saturating at 7 (code = sign << 3 | magnitude, like E2M1's layout);
 *   - block error: SSE = sum of fl(e_i * e_i), e_i = fl(y_i - fl(c_i d)),
 *     summed in fp32 as four sequential runs of 8 (elements 8l..8l+7), then
 *     (P0 + P1) + (P2 + P3); INT4 wins only if its SSE is strictly smaller;
 *   - storage per 32-block: 16 code bytes, two E4M3 scale bytes, one meta
 *     byte (bit 7 = INT4 tag, bits 0-4 = residual position), one bf16. */

double or_int4_decode(uint8_t code)
{
    double m = (double)(code & 7);
    return (code & 8) ? -m : m;
}

uint8_t or_int4_encode(double v)
{
    double a = fabs(v);
    double n = floor(a);
    double f = a - n;
    if (f > 0.5 || (f == 0.5 && fmod(n, 2.0) == 1.0))
        n += 1.0;
    if (n > 7.0)
        n = 7.0;
    return (uint8_t)((signbit(v) ? 8 : 0) | (int)n);
}

static uint16_t f32_to_bf16_bits_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static float bf16_bits_to_f32(uint16_t b) { return bf16_to_f32(b); }

/* One candidate for a 32-block of residual-free rotated values yp[32]:
 * qmax = 6 (E2M1) or 7 (INT4).  Writes codes[32], sb[2]; returns the SSE. */
static float tf4_candidate(const float *yp, float st, int int4, uint8_t *codes,
                           uint8_t *sb)
{
    const float t = (int4 ? 7.0f : 6.0f) * st;
    float err[32];
    for (int h = 0; h < 2; h++) {
        float amax = 0.0f;
        for (int i = 0; i < 16; i++) {
            float a = fabsf(yp[16 * h + i]);
            if (a > amax)
                amax = a;
        }
        uint8_t sc = or_e4m3_encode(amax / t);
        sb[h] = sc;
        float sv = (float)or_e4m3_decode(sc);
        float d = st * sv;
        for (int i = 16 * h; i < 16 * h + 16; i++) {
            uint8_t c;
            float dq;
            if (sv == 0.0f) {
                c = (uint8_t)(signbit(yp[i]) ? 8 : 0);
                dq = 0.0f;
            } else {
                float v = yp[i] / d;
                c = int4 ? or_int4_encode((double)v) : or_e2m1_encode((double)v, 0);
                float cv = (float)(int4 ? or_int4_decode(c) : or_e2m1_decode(c));
                dq = cv * d;
            }
            codes[i] = c;
            err[i] = yp[i] - dq;
        }
    }
    float part[4];
    for (int l = 0; l < 4; l++) {
        float acc = 0.0f;
        for (int i = 8 * l; i < 8 * l + 8; i++) {
            float sq = err[i] * err[i];
            acc = acc + sq;
        }
        part[l] = acc;
    }
    float a01 = part[0] + part[1];
    float a23 = part[2] + part[3];
    return a01 + a23;
}

/* Residual step on one rotated block: position of the largest |y| (lowest
 * index on ties), its bf16 value, and the residual-free block. */
static int tf4_split(const float *y, float *yp, uint16_t *res)
{
    int at = 0;
    float best = fabsf(y[0]);
    for (int i = 1; i < 32; i++)
        if (fabsf(y[i]) > best) {
            best = fabsf(y[i]);
            at = i;
        }
    for (int i = 0; i < 32; i++)
        yp[i] = y[i];
    *res = f32_to_bf16_bits_rne(y[at]);
    yp[at] = 0.0f;
    return at;
}

/* Encode rotated values y[rows][k] (fp32, k % 32 == 0) with tensor scale
 * *gscale (computed from the residual-free values when compute_gscale != 0).
 * Outputs q[rows][k/2], s[rows][k/16] E4M3, meta[rows][k/32],
 * res[rows][k/32] bf16 bits. */
void or_tf4_encode_rotated(const float *y, int64_t rows, int64_t k, float *gscale,
                           int compute_gscale, uint8_t *q, uint8_t *s,
                           uint8_t *meta, uint16_t *res)
{
    const int64_t nb = k / 32;
    if (compute_gscale) {
        float amax = 0.0f;
        for (int64_t r = 0; r < rows; r++)
            for (int64_t b = 0; b < nb; b++) {
                float yp[32];
                uint16_t rv;
                tf4_split(y + r * k + b * 32, yp, &rv);
                for (int i = 0; i < 32; i++)
                    if (fabsf(yp[i]) > amax)
                        amax = fabsf(yp[i]);
            }
        *gscale = or_nv_tensor_scale(amax);
    }
    const float st = *gscale;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            float yp[32];
            uint16_t rv;
            int at = tf4_split(y + r * k + b * 32, yp, &rv);
            uint8_t cn[32], ci[32], sn[2], si[2];
            float en = tf4_candidate(yp, st, 0, cn, sn);
            float ei = tf4_candidate(yp, st, 1, ci, si);
            int use_int4 = ei < en;
            const uint8_t *c = use_int4 ? ci : cn;
            const uint8_t *sc = use_int4 ? si : sn;
            for (int j = 0; j < 16; j++)
                q[r * (k / 2) + b * 16 + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
            s[r * (k / 16) + 2 * b] = sc[0];
            s[r * (k / 16) + 2 * b + 1] = sc[1];
            meta[r * nb + b] = (uint8_t)((use_int4 ? 0x80 : 0) | at);
            res[r * nb + b] = rv;
        }
    }
}

/* TransFP4 quantize of x[rows][k] (dtype): rotate with H_32, then encode. */
void or_tf4_quantize(const void *x, int dtype, int64_t rows, int64_t k, float *gscale,
                     int compute_gscale, uint8_t *q, uint8_t *s, uint8_t *meta,
                     uint16_t *res)
{
    float *y = (float *)malloc((size_t)(rows * k) * sizeof(float));
    or_hadamard_rotate(x, dtype, rows, k, 32, y);
    or_tf4_encode_rotated(y, rows, k, gscale, compute_gscale, q, s, meta, res);
    free(y);
}

/* Rotated-domain reconstruction yh[rows][k] (fp32): y_hat_i = fl(c_i * d_h)
 * with d_h = fl(s_t * E4M3(s_h)) and the codebook the tag selects, plus the
 * bf16 residual at its position (whose code is zero). */
void or_tf4_decode_rotated(const uint8_t *q, const uint8_t *s, const uint8_t *meta,
                           const uint16_t *res, float gscale, int64_t rows, int64_t k,
                           float *yh)
{
    const int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t m = meta[r * nb + b];
            const int int4 = (m & 0x80) != 0, at = m & 31;
            float *v = yh + r * k + b * 32;
            for (int i = 0; i < 32; i++) {
                uint8_t byte = q[r * (k / 2) + b * 16 + i / 2];
                uint8_t c = (i & 1) ? (byte >> 4) : (byte & 15);
                float d = gscale * (float)or_e4m3_decode(s[r * (k / 16) + 2 * b + i / 16]);
                float cv = (float)(int4 ? or_int4_decode(c) : or_e2m1_decode(c));
                v[i] = cv * d;
            }
            v[at] = v[at] + bf16_bits_to_f32(res[r * nb + b]);
        }
    }
}

/* TransFP4 dequantize: x_hat = H^T y_hat per block (H_32 is symmetric and
 * orthonormal, so H^T = H; same fp32 butterfly as the forward rotation). */
void or_tf4_dequantize(const uint8_t *q, const uint8_t *s, const uint8_t *meta,
                       const uint16_t *res, float gscale, int64_t rows, int64_t k,
                       float *xh)
{
    or_tf4_decode_rotated(q, s, meta, res, gscale, rows, k, xh);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < k / 32; b++)
            fwht_block_f32(xh + r * k + b * 32, 32);
}

/* ------------------------------------------------------------------ */
/* Products and metrics                                                */
/* ------------------------------------------------------------------ */

/* Y[i][j] = sum_k A[i][k] * B[j][k] and S[i][j] = sum_k |A[i][k] * B[j][k]|,
 * both accumulated in double, k innermost.  A linear layer y = x W^T. */
void or_gemm_nt(const double *A, const double *B, int64_t m, int64_t n,
                int64_t k, double *Y, double *S)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; i++) {
        for (int64_t j = 0; j < n; j++) {
            double acc = 0.0, sabs = 0.0;
            for (int64_t t = 0; t < k; t++) {
                double p = A[i * k + t] * B[j * k + t];
                acc += p;
                sabs += fabs(p);
            }
            Y[i * n + j] = acc;
            if (S)
                S[i * n + j] = sabs;
        }
    }
}

/* NMSE = ||x - x_hat||^2 / ||x||^2 and cosine similarity [TRANSFP4 sec. 3.2],
 * in double over flattened tensors. */
void or_metrics(const double *x, const double *xh, int64_t n, double *nmse,
                double *cosine)
{
    double se = 0.0, xx = 0.0, hh = 0.0, xh_dot = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double d = x[i] - xh[i];
        se += d * d;
        xx += x[i] * x[i];
        hh += xh[i] * xh[i];
        xh_dot += x[i] * xh[i];
    }
    *nmse = se / xx;
    *cosine = xh_dot / (sqrt(xx) * sqrt(hh));
}
