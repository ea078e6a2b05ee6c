// w4a8.hip -- MXFP8 activations x MXFP4 weights on the CDNA4 block-scaled
// MFMA (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with an E4M3 operand and an E2M1
// operand; the instruction takes each operand's format separately).
//
// Quantization-aware MXFP4 weights with MXFP8 activations are a release
// format of current open models ["Low-precision inference and MXFP4
// quantization" page, Kimi K3]; MXFP8 = FP8 values with one E8M0 scale per
// 1x32 [infra-guide "4.5 FP8 and NVFP4/MXFP4", sec. 4.2].
//
// Operand layout of the instruction for a 32 x 64 tile (lane l, row l % 32,
// half h = l / 32).  E2M1: the lane holds the 32 consecutive k values
// 32 h .. 32 h + 31 -- one MX block -- as 16 bytes (element 2j in the low
// nibble of byte j).  E4M3: the lane holds two runs of 16 k values,
// 16 h .. 16 h + 15 in bytes 0..15 and 32 + 16 h .. 32 + 16 h + 15 in bytes
// 16..31, so each lane carries halves of both blocks.  The scale operand is
// laid out by block for both formats: lane l brings the E8M0 byte of row
// l % 32, block h.  The stored codes are fed unchanged.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

constexpr int kFmtFp8 = 0, kFmtFp4 = 4;  // f8f6f4 operand format codes (E4M3, E2M1)

// Block tile 128 x 128 of four 64 x 64 wave tiles (2 x 2 MFMAs of 32 x 32
// per 64-k step); every wave reads its own fragments from global memory
// (the operands stay L2-resident across the tiles that share them).
template <bool kBf16Out>
__global__ __launch_bounds__(256) void k_w4a8_direct(const uint8_t* __restrict__ aq8,
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
    const int64_t kb = kk + 32 * half;  // block of this lane's scale (and E2M1 run)
    const bool kval = kb < k;            // k is a multiple of 32: kk + 16 half < k always
    i32x8 fa[2], fb[2];
    int sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int64_t ra = row0 + 32 * i + r32;
      if (ra < m) {
        const uint8_t* p = aq8 + ra * k + kk + 16 * half;
        const i32x4 v0 = *(const i32x4*)p;
        const i32x4 v1 = kk + 32 < k ? *(const i32x4*)(p + 32) : (i32x4){};
        fa[i] = (i32x8){v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        sa[i] = kval ? as[ra * ks + kb / 32] : 127;
      } else {
        fa[i] = (i32x8){};
        sa[i] = 127;
      }
      const int64_t rb = col0 + 32 * i + r32;
      if (rb < n && kval) {
        const i32x4 v = *(const i32x4*)(bq + rb * kq + kb / 2);
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
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], kFmtFp8, kFmtFp4, 0,
                                                                      sa[i], 0, sb[j]);
  }

  // lane holds C[row0 + 32 i + 8 (r / 4) + 4 half + r % 4][col0 + 32 j + r32]
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

hipError_t launch_w4a8(const uint8_t* aq8, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                       int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st) {
  dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 127) / 128));
  if (bf16_out)
    hipLaunchKernelGGL(k_w4a8_direct<true>, grid, dim3(256), 0, st, aq8, as, bq, bs, m, n, k, c);
  else
    hipLaunchKernelGGL(k_w4a8_direct<false>, grid, dim3(256), 0, st, aq8, as, bq, bs, m, n, k, c);
  return hipGetLastError();
}

}  // namespace mxq
