// w4a4.hip -- MXFP4 x MXFP4 GEMM on the CDNA4 block-scaled MFMA
// (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with both operands in E2M1).
//
// Native FP4 matrix math needs quantized activations as well as weights
// [infra-guide "4.5 FP8 and NVFP4/MXFP4", sec. 5]; CDNA 4 has
// exponent-block-scaled matrix instructions [TransFP4 page, sec. 5.1].
//
// Operand layout of the instruction (checked on the device against the CPU
// oracle): for a 32 x 64 fp4 tile, lane l holds row l % 32 and the 32
// consecutive k values 32*(l/32)..+32 as 16 bytes (element 2j in the low
// nibble of byte j -- the same packing as the stored codes) plus ONE E8M0
// scale byte.  One lane's k range is therefore exactly one MXFP4 block, and
// the stored codes are fed to the MFMA unchanged.  The 32 x 32 fp32 result
// sits in lane l, column l % 32, rows 8*(r/4) + 4*(l/32) + r%4 of register r.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

// First version: every wave streams its own operand fragments from global
// memory (L2-resident) -- block tile 128 x 128, wave tile 64 x 64 = 2 x 2
// MFMAs per 64-wide k step.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void k_w4a4_direct(const uint8_t* __restrict__ aq,
                                                     const uint8_t* __restrict__ as,
                                                     const uint8_t* __restrict__ bq,
                                                     const uint8_t* __restrict__ bs, int64_t m, int64_t n,
                                                     int64_t k, void* __restrict__ c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t row0 = (int64_t)blockIdx.y * 128 + 64 * wm;
  const int64_t col0 = (int64_t)blockIdx.x * 128 + 64 * wn;
  const int half = lane >> 5, r32 = lane & 31;
  const int64_t kq = k / 2, ks = k / 32;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = (f32x16){};

  for (int64_t kk = 0; kk < k; kk += 64) {
    const int64_t kb = kk + 32 * half;  // this lane's block start
    const bool kval = kb < k;
    i32x8 fa[2], fb[2];
    int sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int64_t ra = row0 + 32 * i + r32;
      if (ra < m && kval) {
        i32x4 v = *(const i32x4*)(aq + ra * kq + kb / 2);
        fa[i] = (i32x8){v.x, v.y, v.z, v.w, 0, 0, 0, 0};
        sa[i] = as[ra * ks + kb / 32];
      } else {
        fa[i] = (i32x8){};
        sa[i] = 127;
      }
      const int64_t rb = col0 + 32 * i + r32;
      if (rb < n && kval) {
        i32x4 v = *(const i32x4*)(bq + rb * kq + kb / 2);
        fb[i] = (i32x8){v.x, v.y, v.z, v.w, 0, 0, 0, 0};
        sb[i] = bs[rb * ks + kb / 32];
      } else {
        fb[i] = (i32x8){};
        sb[i] = 127;
      }
    }
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 4, 4, 0, sa[i], 0,
                                                                      sb[j]);
  }

#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int64_t cc = col0 + 32 * j + r32;
      if (cc >= n) continue;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t rr = row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (rr >= m) continue;
        if (kBf16Out)
          ((uint16_t*)c)[rr * n + cc] = f32_to_bf16_rne(acc[i][j][r]);
        else
          ((float*)c)[rr * n + cc] = acc[i][j][r];
      }
    }
}

hipError_t launch_w4a4(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                       int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st) {
  dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 127) / 128));
  if (bf16_out)
    hipLaunchKernelGGL(k_w4a4_direct<true>, grid, dim3(256), 0, st, aq, as, bq, bs, m, n, k, c);
  else
    hipLaunchKernelGGL(k_w4a4_direct<false>, grid, dim3(256), 0, st, aq, as, bq, bs, m, n, k, c);
  return hipGetLastError();
}

// Zero fill used for products with an empty k.
__global__ void k_zero(uint32_t* y, int64_t nwords) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nwords) y[i] = 0u;
}
__global__ void k_zero16(uint16_t* y, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 0u;
}

hipError_t launch_zero(void* y, int64_t n, bool bf16, hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(k_zero16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (uint16_t*)y, n);
  else
    hipLaunchKernelGGL(k_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (uint32_t*)y, n);
  return hipGetLastError();
}

}  // namespace mxq
