// w4a16.hip -- W4A16 products: 4-bit weights (MXFP4 or NVFP4) times bf16
// activations, fp32 accumulation [infra-guide "4.5 FP8 and NVFP4/MXFP4",
// sec. 4.2 and 5: weight-only 4-bit saves bandwidth, the multiply stays in
// 16 bits].  The weight is dequantized in registers and never written out in
// 16 bits [TransFP4 page, sec. 2.5].
//
// Decode kernel (small m): HBM-bound stream of the packed weight.  Each
// lane owns one 16-byte code chunk = 32 consecutive k of one weight row,
// i.e. exactly one MXFP4 block (two NVFP4 blocks).  The chunk is expanded to
// exact bf16 with the scaled convert instruction (E2M1 * 2^e needs at most
// two significant bits; an NVFP4 s_b * q needs at most six) and fed to the
// 16x16x32 bf16 MFMA with the activations as the other operand:
//   MFMA A (16 x 32): lane l -> activation row m = l % 16, k slots 8*(l/16)..+8
//   MFMA B (32 x 16): lane l -> weight row n = l % 16, same k slots
// A wave covers 16 weight rows x 128 k per step (4 MFMAs per row tile); the
// four waves of a block split k and are summed in LDS in a fixed order, so
// results are deterministic.
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

constexpr int kWaves = 4;

// Expand one lane's 16 code bytes (32 k values) into four bf16x8 MFMA
// operands, operand j holding k values 8j..8j+7.
template <bool kNv>
__device__ __forceinline__ void dequant_chunk(u32x4 c, unsigned sbytes, bf16x8 w[4]) {
  unsigned d[4] = {c.x, c.y, c.z, c.w};
  if (!kNv) {
    float scale = e8m0_as_scale(sbytes & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 0);
      bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 1);
      bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 2);
      bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 3);
      w[j] = (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
  } else {
    // two E4M3 block scales: k 0..15 and k 16..31 of the chunk
    float s0 = e4m3_value(sbytes & 0xFFu), s1 = e4m3_value((sbytes >> 8) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      float sb = j < 2 ? s0 : s1;
      auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[j], 1.0f, 0);
      auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[j], 1.0f, 1);
      auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[j], 1.0f, 2);
      auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[j], 1.0f, 3);
      // s_b * q is exact in fp32 and in bf16 (at most 6 significant bits)
      w[j] = (bf16x8){(__bf16)(p0[0] * sb), (__bf16)(p0[1] * sb), (__bf16)(p1[0] * sb), (__bf16)(p1[1] * sb),
                      (__bf16)(p2[0] * sb), (__bf16)(p2[1] * sb), (__bf16)(p3[0] * sb), (__bf16)(p3[1] * sb)};
    }
  }
}

template <bool kNv, int R, bool kBf16Out>
__global__ __launch_bounds__(256) void k_w4a16_decode(const uint8_t* __restrict__ wq,
                                                      const uint8_t* __restrict__ ws,
                                                      const float* __restrict__ gscale, int64_t n, int64_t k,
                                                      const uint16_t* __restrict__ x, int64_t m,
                                                      void* __restrict__ y) {
  __shared__ f32x4 red[kWaves][R][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * R);
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t nchunks = (k + 127) / 128;
  const int64_t kq = k / 2;                   // code bytes per row
  const int64_t ks = kNv ? k / 16 : k / 32;  // scale bytes per row
  const bool xrow = (m0 + col) < m;
  const uint16_t* xr = x + (m0 + col) * k;

  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; r++) acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int64_t c = wave; c < nchunks; c += kWaves) {
    const int64_t kb = c * 128 + 32 * g;  // first k of this lane's chunk
    const bool kval = kb < k;
    // NVFP4 allows k % 32 == 16: then the last chunk holds only 16 valid k
    const bool khi = kb + 16 < k;
    bf16x8 xf[4];
    if (xrow && kval) {
      const u32x4* xp = (const u32x4*)(xr + kb);
      xf[0] = __builtin_bit_cast(bf16x8, xp[0]);
      xf[1] = __builtin_bit_cast(bf16x8, xp[1]);
      if (khi) {
        xf[2] = __builtin_bit_cast(bf16x8, xp[2]);
        xf[3] = __builtin_bit_cast(bf16x8, xp[3]);
      } else {
        xf[2] = xf[3] = (bf16x8){};
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; j++) xf[j] = (bf16x8){};
    }
    u32x4 codes[R];
    unsigned sc[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int64_t row = n0 + 16 * r + col;
      if (row < n && kval) {
        if (kNv) {
          // rows are only 8-byte aligned when k % 32 == 16
          const u32x2* cp = (const u32x2*)(wq + row * kq + kb / 2);
          u32x2 lo = __builtin_nontemporal_load(cp);
          u32x2 hi = khi ? __builtin_nontemporal_load(cp + 1) : (u32x2){0u, 0u};
          codes[r] = (u32x4){lo.x, lo.y, hi.x, hi.y};
          const uint8_t* sp = ws + row * ks + kb / 16;
          sc[r] = sp[0] | (khi ? ((unsigned)sp[1] << 8) : 0u);
        } else {
          codes[r] = __builtin_nontemporal_load((const u32x4*)(wq + row * kq + kb / 2));
          sc[r] = ws[row * ks + kb / 32];
        }
      } else {
        codes[r] = (u32x4){0u, 0u, 0u, 0u};
        sc[r] = kNv ? 0u : 127u;
      }
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
      bf16x8 wf[4];
      dequant_chunk<kNv>(codes[r], sc[r], wf);
#pragma unroll
      for (int j = 0; j < 4; j++) acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[j], wf[j], acc[r], 0, 0, 0);
    }
  }

#pragma unroll
  for (int r = 0; r < R; r++) red[wave][r][lane] = acc[r];
  __syncthreads();
  const float st = kNv ? *gscale : 1.0f;
  for (int idx = threadIdx.x; idx < R * 64; idx += 256) {
    const int r = idx >> 6, l = idx & 63;
    f32x4 v = red[0][r][l];
#pragma unroll
    for (int w = 1; w < kWaves; w++) v += red[w][r][l];
    const int64_t nn = n0 + 16 * r + (l & 15);
    if (nn >= n) continue;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int64_t mm = m0 + 4 * (l >> 4) + i;
      if (mm >= m) continue;
      float o = kNv ? v[i] * st : v[i];
      if (kBf16Out)
        ((uint16_t*)y)[mm * n + nn] = f32_to_bf16_rne(o);
      else
        ((float*)y)[mm * n + nn] = o;
    }
  }
}

template <bool kNv, int R>
static void launch_decode(const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n, int64_t k,
                          const void* x, int64_t m, void* y, bool bf16_out, hipStream_t st) {
  dim3 grid((unsigned)((n + 16 * R - 1) / (16 * R)), (unsigned)((m + 15) / 16));
  if (bf16_out)
    hipLaunchKernelGGL((k_w4a16_decode<kNv, R, true>), grid, dim3(256), 0, st, wq, ws, gscale, n, k,
                       (const uint16_t*)x, m, y);
  else
    hipLaunchKernelGGL((k_w4a16_decode<kNv, R, false>), grid, dim3(256), 0, st, wq, ws, gscale, n, k,
                       (const uint16_t*)x, m, y);
}

hipError_t launch_w4a16(bool nv, const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n,
                        int64_t k, const void* x, int64_t m, void* y, bool bf16_out, hipStream_t st) {
  if (nv)
    launch_decode<true, 2>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  else
    launch_decode<false, 2>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  return hipGetLastError();
}

}  // namespace mxq
