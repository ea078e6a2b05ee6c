// mxq_launch.h -- host-side launchers of the library's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace mxq {

hipError_t launch_mx_quantize(const void* x, bool bf16, int64_t rows, int64_t k, uint8_t* q, uint8_t* s,
                              hipStream_t st);
// MXFP8: q[rows][k] E4M3 codes, s[rows][k/32] E8M0 codes.
hipError_t launch_mx8_quantize(const void* x, bool bf16, int64_t rows, int64_t k, uint8_t* q, uint8_t* s,
                               hipStream_t st);
// W4A8: c[m][n] = sum_k A8_hat[m][k] * B4_hat[n][k], A MXFP8 (aq8[m][k],
// as[m][k/32]), B MXFP4; fp32 accumulation; c as fp32 or bf16.
hipError_t launch_w4a8(const uint8_t* aq8, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                       int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st);
// MXFP4 of x rotated block by block along k with the orthonormal Hadamard
// H_hk, hk in {16, 32, 64, 128}, k % max(32, hk) == 0.
hipError_t launch_mx_quantize_hadamard(const void* x, bool bf16, int64_t rows, int64_t k, int hk, uint8_t* q,
                                       uint8_t* s, hipStream_t st);
hipError_t launch_mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t k, void* y,
                                bool bf16, hipStream_t st);
hipError_t launch_nv_quantize(const void* x, bool bf16, int64_t rows, int64_t k, float* gscale,
                              bool compute_gscale, uint8_t* q, uint8_t* s, hipStream_t st);
hipError_t launch_tf4_quantize(const void* x, bool bf16, int64_t rows, int64_t k, float* gscale,
                               bool compute_gscale, uint8_t* q, uint8_t* s, uint8_t* meta, uint16_t* res,
                               hipStream_t st);
hipError_t launch_tf4_dequantize(const uint8_t* q, const uint8_t* s, const uint8_t* meta, const uint16_t* res,
                                 const float* gscale, int64_t rows, int64_t k, void* y, bool bf16_out,
                                 hipStream_t st);
hipError_t launch_nv_dequantize(const uint8_t* q, const uint8_t* s, const float* gscale, int64_t rows,
                                int64_t k, void* y, bool bf16, hipStream_t st);

// W4A16: y[m][n] = (gscale ? *gscale : 1) * sum_k x[m][k] * deq(W)[n][k].
// nv == false: MXFP4 weight (E8M0 per 32); nv == true: NVFP4 (E4M3 per 16).
hipError_t launch_w4a16(bool nv, const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n,
                        int64_t k, const void* x, int64_t m, void* y, bool bf16_out, hipStream_t st);

// W4A4: c[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k] on the block-scaled MFMA.
hipError_t launch_w4a4(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                       int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st);

// W4A4 and W4A8 for few activation rows (weight-stream bound), used where
// gemm_skinny_applies: m <= 128, k % 512 == 0, k <= 2^24.
bool gemm_skinny_applies(int64_t m, int64_t k);
hipError_t launch_w4a4_skinny(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                              int64_t m, int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st);
hipError_t launch_w4a8_skinny(const uint8_t* aq8, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                              int64_t m, int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st);
// W4A4 with bf16 activations x[m][k] quantized to MXFP4 inside the kernel:
// bit-identical to launch_mx_quantize followed by launch_w4a4.  For
// 1 <= m <= 16 where gemm_skinny_applies.
hipError_t launch_w4a4_dynamic(const uint16_t* x, const uint8_t* bq, const uint8_t* bs, int64_t m, int64_t n,
                               int64_t k, void* c, bool bf16_out, hipStream_t st);
// W4A8 with bf16 activations quantized to MXFP8 inside the kernel:
// bit-identical to launch_mx8_quantize followed by launch_w4a8.  For
// 1 <= m <= 16 where gemm_skinny_applies.
hipError_t launch_w4a8_dynamic(const uint16_t* x, const uint8_t* bq, const uint8_t* bs, int64_t m, int64_t n,
                               int64_t k, void* c, bool bf16_out, hipStream_t st);

// W4A4 with the product rounded to bf16 and quantized to MXFP4 along n in
// the epilogue: cq[m][n/2], cs[m][n/32]; n % 32 == 0.
hipError_t launch_w4a4_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                          int64_t n, int64_t k, uint8_t* cq, uint8_t* cs, hipStream_t st);

}  // namespace mxq
