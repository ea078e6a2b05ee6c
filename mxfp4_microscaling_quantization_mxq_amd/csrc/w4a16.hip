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
// One "chunk" step of a wave covers 16 weight rows x 128 k (4 MFMAs per row
// tile).  A wave keeps R row tiles x U chunks of loads in flight (all issued
// before the first is consumed, with no branches in between), which is what
// it takes to cover HBM latency.  The waves of a block split k round-robin
// by chunk and are summed in LDS in a fixed order: deterministic results.
#include <type_traits>

#include "mxq_device.h"
#include "mxq_gemm_common.h"
#include "mxq_launch.h"

namespace mxq {

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
    const float s0 = e4m3_value_b<0>(sbytes), s1 = e4m3_value_b<1>(sbytes);
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

// Loads of one lane for one (row tile, chunk): 16 code bytes and the scale
// byte(s).  Invalid lanes read a valid dummy address and are zeroed by a
// select, so the load sequence has no branches.  kWide: NVFP4 rows known to
// be 16-byte aligned (k % 32 == 0) and the chunk whole, one 16-byte load.
template <bool kNv, bool kLoadScale = true, bool kWide = false>
__device__ __forceinline__ void load_chunk(const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws,
                                           int64_t row, int64_t kb, bool valid, bool khi, int64_t kq, int64_t ks,
                                           u32x4& codes, unsigned& sc) {
  static_assert(!(kNv && kWide && kLoadScale), "the wide NVFP4 load takes its scales from the staged copy");
  const int64_t r = valid ? row : 0;
  const int64_t b = valid ? kb : 0;
  if (!kNv || kWide) {
    u32x4 c = __builtin_nontemporal_load((const u32x4*)(wq + r * kq + b / 2));
    codes = valid ? c : (u32x4){0u, 0u, 0u, 0u};
    if (kLoadScale) {
      unsigned s = ws[r * ks + b / 32];
      sc = valid ? s : 127u;
    }
  } else {
    // rows are only 8-byte aligned when k % 32 == 16; the second half of the
    // chunk exists only if kb + 16 < k
    const bool hi = valid && khi;
    const u32x2* cp = (const u32x2*)(wq + r * kq + b / 2);
    u32x2 lo = __builtin_nontemporal_load(cp);
    u32x2 h2 = __builtin_nontemporal_load(hi ? cp + 1 : cp);
    const uint8_t* sp = ws + r * ks + b / 16;
    unsigned s0 = sp[0];
    unsigned s1 = sp[hi ? 1 : 0];
    codes = valid ? (u32x4){lo.x, lo.y, hi ? h2.x : 0u, hi ? h2.y : 0u} : (u32x4){0u, 0u, 0u, 0u};
    sc = valid ? (s0 | (hi ? s1 << 8 : 0u)) : 0u;
  }
}

template <bool kNv, int R, int U, int W, bool kBf16Out>
__global__ __launch_bounds__(64 * W) void k_w4a16_decode(const uint8_t* __restrict__ wq,
                                                         const uint8_t* __restrict__ ws,
                                                         const float* __restrict__ gscale, int64_t n, int64_t k,
                                                         const uint16_t* __restrict__ x, int64_t m,
                                                         void* __restrict__ y) {
  __shared__ f32x4 red[W][R][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * R);
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t nchunks = (k + 127) / 128;
  const int64_t kq = k / 2;                   // code bytes per row
  const int64_t ks = kNv ? k / 16 : k / 32;  // scale bytes per row
  const bool xrow = (m0 + col) < m;
  const uint16_t* xr = x + (xrow ? (m0 + col) : 0) * k;

  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; r++) acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int64_t c0 = wave; c0 < nchunks; c0 += W * U) {
    u32x4 codes[U][R];
    unsigned sc[U][R];
    bf16x8 xf[U][4];
    // ---- issue every load of this step
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t kb = (c0 + (int64_t)W * u) * 128 + 32 * g;  // first k of the lane's chunk
      const bool kval = kb < k;
      const bool khi = kb + 16 < k;
#pragma unroll
      for (int r = 0; r < R; r++) {
        const int64_t row = n0 + 16 * r + col;
        load_chunk<kNv>(wq, ws, row, kb, kval && row < n, khi, kq, ks, codes[u][r], sc[u][r]);
      }
      const bool xv = xrow && kval;
      const u32x4* xp = (const u32x4*)(xr + (xv ? kb : 0));
      const bool xhi = xv && khi;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        u32x4 v = xp[(j < 2 || xhi) ? j : 0];
        const bool ok = j < 2 ? xv : xhi;
        xf[u][j] = __builtin_bit_cast(bf16x8, ok ? v : (u32x4){0u, 0u, 0u, 0u});
      }
    }
    // ---- consume
#pragma unroll
    for (int u = 0; u < U; u++) {
#pragma unroll
      for (int r = 0; r < R; r++) {
        bf16x8 wf[4];
        dequant_chunk<kNv>(codes[u][r], sc[u][r], wf);
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[u][j], wf[j], acc[r], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; r++) red[wave][r][lane] = acc[r];
  __syncthreads();
  const float st = kNv ? *gscale : 1.0f;
  for (int idx = threadIdx.x; idx < R * 64; idx += 64 * W) {
    const int r = idx >> 6, l = idx & 63;
    f32x4 v = red[0][r][l];
#pragma unroll
    for (int w = 1; w < W; w++) v += red[w][r][l];
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

// ---------------------------------------------------------------------------
// Decode kernel for m <= 4 (vector ALU).  HBM efficiency decides this path:
// each wave load instruction reads 1 KiB of ONE weight row (lane l: the 16
// code bytes of k = kr*2048 + 32l .. +32, plus that block's scale byte), the
// same access pattern as a linear stream.  Lane l keeps the activations of
// its 32 k values in registers for the whole row sweep; per row it expands
// its codes to exact (unscaled) E2M1 values in bf16 and accumulates
// v_dot2_f32_bf16 products, then applies the block scale with one fp32 FMA
// (MXFP4: 2^e, exact; NVFP4: the E4M3 block scale, per 16).  MXFP4 with one
// activation row instead folds the scale into the convert and takes the dot
// products off the vector ALU onto the MFMA (the diagonal form below).  Each
// lane ends with one partial sum per (activation row, weight row); the 64
// lanes x W waves are summed through LDS in a fixed order.
// MXFP4, one activation row: dot products on the MFMA diagonal (1) or with
// v_dot2_f32_bf16 (0).  Interleaved A/B on 28672 x 8192: 23.35-24.15 against
// 23.89-24.85 us, 63 of 63 parity cases on both.
#ifndef MXQ_DV_MFMA1
#define MXQ_DV_MFMA1 1
#endif
template <bool kNv, int M, int RB, int U, int W, bool kBf16Out>
__global__ __launch_bounds__(64 * W) void k_w4a16_decode_valu(const uint8_t* __restrict__ wq,
                                                              const uint8_t* __restrict__ ws,
                                                              const float* __restrict__ gscale, int64_t n,
                                                              int64_t k, const uint16_t* __restrict__ x,
                                                              void* __restrict__ y) {
  static_assert(RB % U == 0, "rows per block must be a multiple of the unroll");
  // MXFP4 at one activation row: dot products on the MFMA (see below)
  constexpr bool kDiagMfma = !kNv && M == 1 && MXQ_DV_MFMA1;
  const int de = threadIdx.x & 3;                                        // diagonal element
  const bool ddiag = ((threadIdx.x & 15) >> 2) == ((threadIdx.x & 63) >> 4);  // lane holds one
  // per-wave partial sums: red[wave][act row][weight row][lane]
  __shared__ float red[W][M][RB][64];
  // Scale bytes of a wave's 8 rows for its 2048-k range (64 MXFP4 or 128
  // NVFP4 blocks per row), fetched with one 8- or 16-byte-per-lane load
  // instead of eight 1- or 2-byte-per-lane loads (those small requests cost
  // about 10 % of the MXFP4 decode time)
  constexpr int SB = kNv ? 128 : 64;  // scale bytes per row per range
  __shared__ __attribute__((aligned(16))) uint8_t sstage[W][8][SB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches and offsets
  const int64_t n0 = (int64_t)blockIdx.x * RB;
  const int64_t kq = k / 2;                   // code bytes per row
  const int64_t ks = kNv ? k / 16 : k / 32;  // scale bytes per row
  const int64_t nkr = (k + 2047) / 2048;      // k ranges of 64 lanes x 32

  for (int mm = 0; mm < M; mm++)
    for (int r = 0; r < RB; r++) red[wave][mm][r][lane] = 0.f;

  // MXFP4 with one k range per wave (6144 < k <= 8192, k % 256 == 0) and a
  // whole block of rows: the scale bytes of the block's rows are one
  // contiguous RB x ks stretch, read block-wide in full 128-byte lines
  // (each wave's own 64-byte slices per row made half-line requests, which
  // move half the bytes per request).  Block-uniform, so every wave meets
  // the barrier below exactly once.
  __shared__ __attribute__((aligned(16))) uint8_t sblk[kNv ? 16 : RB * 256];
  const bool blk_sc = !kNv && U % 8 == 0 && RB % 8 == 0 && nkr == W && k % 256 == 0 && n0 + RB <= n;

  for (int64_t kr = wave; kr < nkr; kr += W) {
    const int64_t kb = kr * 2048 + 32 * lane;  // this lane's 32 k values
    const bool kval = kb < k;
    const bool khi = kb + 16 < k;  // NVFP4 may end on a half chunk
    // activations of this lane's k values: 16 bf16 pairs per activation row
    bf16x2 xs[M][16];
#pragma unroll
    for (int mm = 0; mm < M; mm++) {
      const bf16x8* xp = (const bf16x8*)(x + mm * k + (kval ? kb : 0));
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const bool ok = kval && (j < 2 || khi);
        bf16x8 v = xp[ok ? j : 0];
#pragma unroll
        for (int p = 0; p < 4; p++)
          xs[mm][4 * j + p] = ok ? (bf16x2){v[2 * p], v[2 * p + 1]} : (bf16x2){(__bf16)0.f, (__bf16)0.f};
      }
    }
#pragma unroll 1
    for (int r0 = 0; r0 < RB; r0 += U) {
      u32x4 codes[U];
      unsigned sc[U];
      // fast scale path: 8 rows per step, this wave's 2048-k range whole
      // and every row's scale segment aligned to the per-lane load (8 B
      // MXFP4, 16 B NVFP4; NVFP4 rows are then 16-byte aligned too)
      const bool stage_sc = U == 8 && (kr + 1) * SB <= ks && ks % (SB / 8) == 0;
      if (blk_sc) {
        // the block's RB x ks scale bytes, contiguous, in full-line loads
        // (one or two 8-byte pieces per thread) staged in LDS once, before
        // the first rows' codes are consumed
        u32x2 piece[RB / 8];
        if (r0 == 0) {
#pragma unroll
          for (int p = 0; p < RB / 8; p++) {
            const int64_t off = 8 * ((int64_t)threadIdx.x + 64 * W * p);
            piece[p] = off < RB * ks ? *(const u32x2*)(ws + n0 * ks + off) : (u32x2){0u, 0u};
          }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int64_t row = n0 + r0 + u;
          load_chunk<kNv, false, kNv>(wq, ws, row, kb, kval && row < n, khi, kq, ks, codes[u], sc[u]);
        }
        if (r0 == 0) {
#pragma unroll
          for (int p = 0; p < RB / 8; p++) {
            const int off = 8 * (threadIdx.x + 64 * W * p);
            if (off < RB * ks) *(u32x2*)&sblk[off] = piece[p];
          }
          __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < U; u++) sc[u] = kval ? (unsigned)sblk[(r0 + u) * ks + kr * 64 + lane] : 127u;
      } else if (stage_sc) {
        const int rr = lane >> 3;
        const int64_t srow = n0 + r0 + rr;
        const uint8_t* sp = ws + (srow < n ? srow : 0) * ks + kr * SB + (SB / 8) * (lane & 7);
        u32x4 sv;
        if (kNv) {
          sv = *(const u32x4*)sp;
        } else {
          const u32x2 s2 = *(const u32x2*)sp;
          sv = (u32x4){s2.x, s2.y, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int64_t row = n0 + r0 + u;
          load_chunk<kNv, false, kNv>(wq, ws, row, kb, kval && row < n, khi, kq, ks, codes[u], sc[u]);
        }
        if (kNv)
          *(u32x4*)&sstage[wave][rr][16 * (lane & 7)] = sv;
        else
          *(u32x2*)&sstage[wave][rr][8 * (lane & 7)] = (u32x2){sv.x, sv.y};
        // the wave reads back what it wrote: one wave's LDS operations run in
        // order.  NVFP4: the lane's two blocks (halves of its 32 k) as one
        // 16-bit pair, low byte first.
#pragma unroll
        for (int u = 0; u < U; u++) {
          const bool v = n0 + r0 + u < n;
          if (kNv)
            sc[u] = v ? (unsigned)*(const uint16_t*)&sstage[wave][u][2 * lane] : 0u;
          else
            sc[u] = v ? (unsigned)sstage[wave][u][lane] : 127u;
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int64_t row = n0 + r0 + u;
          load_chunk<kNv>(wq, ws, row, kb, kval && row < n, khi, kq, ks, codes[u], sc[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const unsigned d[4] = {codes[u].x, codes[u].y, codes[u].z, codes[u].w};
        if constexpr (kDiagMfma) {
          // MXFP4, one activation row: the lane's 32 codes are one block, so
          // its scale rides in the convert (exact bf16, as in the ring), and
          // the 16x16x32 MFMA of the lanes' weight fragments (A: lane (g, c)
          // gives row c, k 8g..8g+7) with their activation fragments at the
          // same k (B: column c) has on its diagonal D[c][c] the dot product
          // of lanes c, 16 + c, 32 + c, 48 + c.  Off-diagonal entries pair
          // different lanes' k and are dropped; lane (g, 4g + e) holds
          // D[4g + e][4g + e] as element e.  One convert per two weights and
          // four MFMAs replace the dot products and the scale multiply.
          const float scale = e8m0_as_scale(sc[u] & 0xFFu);
          f32x4 dm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 0);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 1);
            const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 2);
            const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 3);
            const bf16x8 wa = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            const bf16x8 xb = {xs[0][4 * j][0], xs[0][4 * j][1], xs[0][4 * j + 1][0], xs[0][4 * j + 1][1],
                               xs[0][4 * j + 2][0], xs[0][4 * j + 2][1], xs[0][4 * j + 3][0], xs[0][4 * j + 3][1]};
            dm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb, dm, 0, 0, 0);
          }
          float dv = dm[0];
          dv = de == 1 ? dm[1] : dv;
          dv = de == 2 ? dm[2] : dv;
          dv = de == 3 ? dm[3] : dv;
          red[wave][0][r0 + u][lane] += ddiag ? dv : 0.f;
          continue;
        }
        bf16x2 w[16];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          w[4 * j + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], 1.0f, 0);
          w[4 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], 1.0f, 1);
          w[4 * j + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], 1.0f, 2);
          w[4 * j + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], 1.0f, 3);
        }
#pragma unroll
        for (int mm = 0; mm < M; mm++) {
          float acc = red[wave][mm][r0 + u][lane];
          if (!kNv) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < 16; i++) p = __builtin_amdgcn_fdot2_f32_bf16(w[i], xs[mm][i], p, false);
            acc = __builtin_fmaf(p, e8m0_value(sc[u] & 0xFFu), acc);
          } else {
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) p0 = __builtin_amdgcn_fdot2_f32_bf16(w[i], xs[mm][i], p0, false);
#pragma unroll
            for (int i = 8; i < 16; i++) p1 = __builtin_amdgcn_fdot2_f32_bf16(w[i], xs[mm][i], p1, false);
            acc = __builtin_fmaf(p0, e4m3_value_b<0>(sc[u]), acc);
            acc = __builtin_fmaf(p1, e4m3_value_b<1>(sc[u]), acc);
          }
          red[wave][mm][r0 + u][lane] = acc;
        }
      }
    }
  }
  __syncthreads();
  // sum of W x 64 partials per output, 8 threads per output, fixed order
  const float st = kNv ? *gscale : 1.0f;
  for (int o = threadIdx.x >> 3; o < M * RB; o += 8 * W) {
    const int part = threadIdx.x & 7;
    const int mm = o / RB, r = o % RB;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < W; w++)
#pragma unroll
      for (int i = 0; i < 8; i++) v += red[w][mm][r][part * 8 + i];
    v += __shfl_xor(v, 1, 8);
    v += __shfl_xor(v, 2, 8);
    v += __shfl_xor(v, 4, 8);
    const int64_t nn = n0 + r;
    if (part == 0 && nn < n) {
      const float out = kNv ? v * st : v;
      if (kBf16Out)
        ((uint16_t*)y)[mm * n + nn] = f32_to_bf16_rne(out);
      else
        ((float*)y)[mm * n + nn] = out;
    }
  }
}

// m = 1: weight rows per block and rows whose loads a wave issues at once
#ifndef MXQ_DV_RB1
#define MXQ_DV_RB1 8
#define MXQ_DV_U1 8
#endif
template <bool kNv, int M>
static void launch_decode_valu(const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n, int64_t k,
                               const void* x, void* y, bool bf16_out, hipStream_t st) {
  constexpr int RB = M == 1 ? MXQ_DV_RB1 : 16, U = M == 1 ? MXQ_DV_U1 : 8, W = 4;
  dim3 grid((unsigned)((n + RB - 1) / RB));
  if (bf16_out)
    hipLaunchKernelGGL((k_w4a16_decode_valu<kNv, M, RB, U, W, true>), grid, dim3(64 * W), 0, st, wq, ws, gscale,
                       n, k, (const uint16_t*)x, y);
  else
    hipLaunchKernelGGL((k_w4a16_decode_valu<kNv, M, RB, U, W, false>), grid, dim3(64 * W), 0, st, wq, ws, gscale,
                       n, k, (const uint16_t*)x, y);
}

// ---------------------------------------------------------------------------
// Decode kernel for 2 <= m <= 16 (MXFP4, bf16 MFMA).  Same row-contiguous
// weight stream as the vector-ALU kernel -- each wave load instruction reads
// 1 KiB of one row (lane l: 16 code bytes of k = kr*2048 + 32 l .. +32) and
// the row's 64 scale bytes for that range -- but the arithmetic is the
// 16x16x32 bf16 MFMA, whose cost does not grow with m.
//   * a wave owns 16 weight rows for the whole k; the block (4 waves, 64
//     rows) walks k in ranges of 2048;
//   * per range the block stages the activation slice x[0..m)[range] in LDS
//     once (shared by the four waves), and each wave writes its 16 x 1 KiB
//     code tile to its own LDS region (rows padded by 16 B) and reads it back
//     in the MFMA operand layout: lane (col, g) takes row col, 32-k block
//     4c + g of chunk c, dequantized in registers as in the tiled kernel;
//   * the next range's codes, scales and activations are loaded into
//     registers while the current range is multiplied.
// Each wave's 16 x 16 accumulator covers all of k: no cross-wave sum.
constexpr int kDRow = 1024 + 16;  // LDS pitch of one 1 KiB code row
constexpr int kXRow = 4096 + 16;  // LDS pitch of one activation row slice (2048 bf16)

template <bool kBf16Out>
__global__ __launch_bounds__(256) void k_w4a16_decode_mfma(const uint8_t* __restrict__ wq,
                                                           const uint8_t* __restrict__ ws, int64_t n, int64_t k,
                                                           const uint16_t* __restrict__ x, int64_t m,
                                                           void* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t codes_lds[4][16 * kDRow];
  __shared__ uint8_t scale_lds[4][16][64];
  __shared__ __attribute__((aligned(16))) uint8_t x_lds[16 * kXRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t nw0 = (int64_t)blockIdx.x * 64 + 16 * wave;  // this wave's first row
  const int64_t kq = k / 2, ks = k / 32;
  const int nkr = (int)((k + 2047) / 2048);
  uint8_t* cl = codes_lds[wave];
  const int xm = (int)min((int64_t)col, m - 1);  // activation row of this lane

  // register staging of one range: 16 code chunks + 16 scale bytes per
  // lane, and up to 16 activation pieces of 16 B per thread
  u32x4 c[16];
  unsigned sc[16];
  u32x4 xv[16];
  auto load_range = [&](int kr) {
    const int64_t kb = (int64_t)kr * 2048 + 32 * lane;
    const bool kval = kb < k;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t row = nw0 + r;
      const bool v = kval && row < n;
      const int64_t rr = v ? row : 0, bb = v ? kb : 0;
      u32x4 t = __builtin_nontemporal_load((const u32x4*)(wq + rr * kq + bb / 2));
      unsigned sv = ws[rr * ks + bb / 32];
      c[r] = v ? t : (u32x4){0u, 0u, 0u, 0u};
      sc[r] = v ? sv : 127u;
    }
    // activation slice: m rows x 4 KiB, 16 B per thread per row
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int64_t kk = (int64_t)kr * 2048 + 8 * tid;
      const bool v = r < m && kk < k;
      const u32x4 t = *(const u32x4*)(x + (v ? r * k + kk : 0));
      xv[r] = v ? t : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto store_range = [&]() {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      *(u32x4*)(cl + r * kDRow + 16 * lane) = c[r];
      scale_lds[wave][r][lane] = (uint8_t)sc[r];
    }
#pragma unroll
    for (int r = 0; r < 16; r++)
      if (r < m) *(u32x4*)(x_lds + r * kXRow + 16 * tid) = xv[r];
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  load_range(0);
  for (int kr = 0; kr < nkr; kr++) {
    store_range();
    __syncthreads();  // activation slice and code tiles in LDS
    if (kr + 1 < nkr) load_range(kr + 1);
    const int nch = (int)min((int64_t)16, (k - (int64_t)kr * 2048 + 127) / 128);
    for (int ch = 0; ch < nch; ch++) {
      const int blk = 4 * ch + g;  // this lane's 32-k block within the range
      const u32x4 cw = *(const u32x4*)(cl + col * kDRow + blk * 16);
      const float scale = e8m0_as_scale(scale_lds[wave][col][blk]);
      const bf16x8* xp = (const bf16x8*)(x_lds + xm * kXRow + blk * 64);
      const unsigned d[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 0);
        bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 1);
        bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 2);
        bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], scale, 3);
        const bf16x8 wf = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xp[j], wf, acc, 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done reading before the next range lands
  }
  // lane holds y[4g + i][nw0 + col]
  const int64_t nn = nw0 + col;
  if (nn < n) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int64_t mm = 4 * g + i;
      if (mm >= m) continue;
      if (kBf16Out)
        ((uint16_t*)y)[mm * n + nn] = f32_to_bf16_rne(acc[i]);
      else
        ((float*)y)[mm * n + nn] = acc[i];
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM kernel (large m, k % 64 == 0): bf16 MFMA, MFMA-bound.
// Block tile 256 (x rows) x 256 (weight rows), eight waves of 128 x 64 (or
// four of 128 x 128), each a grid of v_mfma_f32_32x32x16_bf16 per 16-k step.
// k advances in stages of 64 through a ring of three LDS stages filled by
// direct buffer -> LDS loads (buffer_load_dwordx4 ... lds):
//   * x: 256 rows x 128 B per stage, 16-B unit u of row r stored at
//     u ^ ((r >> 1) & 7) (conflict-free fragment reads);
//   * weight codes: 256 rows x 32 B per stage, unit u at u ^ ((r >> 3) & 1).
// MFMA k slots are permuted so that a lane's 8 k values of step kk are
// k = 32*half + 8*kk + 0..7: its weight codes for the whole stage are then
// one 16-B chunk = one MXFP4 block (two NVFP4 blocks), dequantized per step
// in registers -- MXFP4 with the scaled convert (exact bf16), NVFP4 as
// E4M3 * E2M1 in fp32 (exact, <= 6 significant bits) -- and x is read with
// the same permutation.  Operands are swapped (weight rows on the
// instruction's A side) so a lane stores four consecutive outputs at once.
// The NVFP4 tensor scale multiplies the fp32 result in the epilogue.
constexpr int kGBM = 256, kGBN = 256, kGRing = 3;
constexpr int kGXStage = kGBM * 128, kGWStage = kGBN * 32;
// One ring slot of the GEMM (activations and weight codes of one stage).
// Every slot is its own LDS variable and is addressed only through
// compile-time slot indices, so the compiler can tell that the reads of one
// slot do not touch the slots whose copies are in flight.
struct GSlot {
  uint8_t x[kGXStage];
  uint8_t w[kGWStage];
};
template <int B>
__device__ __forceinline__ GSlot& g_slot() {
  __shared__ __attribute__((aligned(1024))) GSlot slot;
  return slot;
}

// NWV waves per block in a WNR x (NWV / WNR) grid: 4 waves as 2 x 2 tiles
// of 128 x 128 (one wave per SIMD), 8 as 2 x 4 of 128 x 64 (two waves per
// SIMD, so one wave's MFMAs cover the other's fragment reads, expansion and
// waits), or 8 as 1 x 8 of 256 x 32: every weight fragment then has a single
// wave expanding it (in 2 x 4 the two waves of a SIMD expand the same
// fragments), at twice the activation fragment reads -- the trade NVFP4's
// per-element E4M3 multiply makes worthwhile.
template <bool kNv, bool kBf16Out, int NWV, int WNR>
__global__ __launch_bounds__(64 * NWV, 1) void k_w4a16_gemm(const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws,
                                                       const float* __restrict__ gscale, int64_t n, int64_t k,
                                                       const uint16_t* __restrict__ x, int64_t m,
                                                       void* __restrict__ y) {
  static_assert((NWV == 4 && WNR == 2) || (NWV == 8 && (WNR == 2 || WNR == 1)), "wave grid");
  constexpr int WNC = NWV / WNR;       // wave columns
  constexpr int WROWS = kGBM / WNR;    // activation rows per wave
  constexpr int IA = WROWS / 32;       // activation fragments per wave
  constexpr int WCOLS = kGBN / WNC;    // weight rows (output columns) per wave
  constexpr int JB = WCOLS / 32;       // weight fragments per wave
  constexpr int RPW = kGBM / NWV;      // rows of x and of W each wave copies
  constexpr int CJX = RPW / 8;         // x copies per wave per stage (8 rows of 128 B each)
  constexpr int CJW = RPW / 32;        // weight copies per wave per stage (32 rows of 32 B each)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNC, wn = wave % WNC;
  const int half = lane >> 5, r32 = lane & 31;

  const int64_t tm_n = (m + kGBM - 1) / kGBM, tn_n = (n + kGBN - 1) / kGBN;
  const int64_t tiles = tm_n * tn_n;
  int64_t tl = blockIdx.x;
  if (tiles % 8 == 0) tl = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int64_t per_group = 4 * tn_n;
  const int64_t g0 = (tl / per_group) * 4;
  const int64_t gsz = (tm_n - g0) < 4 ? (tm_n - g0) : 4;
  const int64_t m0 = (g0 + (tl % per_group) % gsz) * kGBM;
  const int64_t n0 = ((tl % per_group) / gsz) * kGBN;
  const int rows_x = (int)min((int64_t)kGBM, m - m0), rows_w = (int)min((int64_t)kGBN, n - n0);

  const int64_t kq = k / 2, ks = kNv ? k / 16 : k / 32, kx = k * 2;
  const int nstages = (int)(k / 64);

  // CJX + CJW DMA instructions per wave per stage (10 with 4 waves, 5 with 8)
  // stage s into ring slot b (near the end the stage index is clamped to the
  // last stage so every step issues the same number of loads; the copy lands
  // in the free slot and is never read)
  // buffer resources of the tile's row panels; per-lane offsets fixed for
  // the whole k loop, the stage moves the uniform offset only
  const __amdgpu_buffer_rsrc_t rx = panel_rsrc((const uint8_t*)x + m0 * kx, rows_x * kx);
  const __amdgpu_buffer_rsrc_t rw = panel_rsrc(wq + n0 * kq, rows_w * kq);
  unsigned offx[CJX], offw[CJW];
#pragma unroll
  for (int j = 0; j < CJX; j++) {
    // (row >> 1) & 7 == (4 j + lane / 16) & 7: RPW * wave / 2 is a multiple of 8
    const int row = RPW * wave + 8 * j + (lane >> 3);
    const unsigned cu16 = (unsigned)(((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)) << 4);
    offx[j] = (unsigned)min(row, rows_x - 1) * (unsigned)kx + cu16;
  }
#pragma unroll
  for (int j = 0; j < CJW; j++) {
    const int row = RPW * wave + 32 * j + (lane >> 1);
    const unsigned cu16 = (unsigned)(((lane & 1) ^ ((row >> 3) & 1)) << 4);
    offw[j] = (unsigned)min(row, rows_w - 1) * (unsigned)kq + cu16;
  }
  auto issue = [&](auto slot_tag, int s) {
    uint8_t* xb = g_slot<decltype(slot_tag)::value>().x;
    uint8_t* wb = g_slot<decltype(slot_tag)::value>().w;
#pragma unroll
    for (int j = 0; j < CJX; j++) bdma16(rx, offx[j], (unsigned)s * 128u, xb + (RPW * wave + 8 * j) * 128);
#pragma unroll
    for (int j = 0; j < CJW; j++) bdma16(rw, offw[j], (unsigned)s * 32u, wb + (RPW * wave + 32 * j) * 32);
  };
  // this lane's scale byte(s) for its four weight rows at stage s (global,
  // L2-resident): MXFP4 block 2s + half; NVFP4 blocks 4s + 2 half + {0, 1}
  auto load_scales = [&](int s, unsigned sc[JB]) {
#pragma unroll
    for (int j = 0; j < JB; j++) {
      const int64_t row = min(n0 + wn * WCOLS + j * 32 + r32, n - 1);
      if (kNv) {
        const uint8_t* p = ws + row * ks + 4 * (int64_t)s + 2 * half;
        sc[j] = p[0] | ((unsigned)p[1] << 8);
      } else {
        sc[j] = ws[row * ks + 2 * (int64_t)s + half];
      }
    }
  };

  f32x16 acc[IA][JB];
#pragma unroll
  for (int i = 0; i < IA; i++)
#pragma unroll
    for (int j = 0; j < JB; j++) acc[i][j] = (f32x16){};

  const int swz = (r32 >> 1) & 7;
  const int laneX = (wm * WROWS + r32) * 128;
  const int laneW = (wn * WCOLS + r32) * 32 + ((half ^ ((r32 >> 3) & 1)) << 4);

  // weight operands of k step kk from the stage's code chunks: MXFP4 with
  // the scaled convert (exact bf16), NVFP4 as E4M3 * E2M1 in fp32 (exact,
  // at most 6 significant bits) rounded to bf16 (exact)
  auto dequant = [&](const u32x4 wc[JB], int kk, const unsigned sc[JB], bf16x8 wf[JB]) {
#pragma unroll
    for (int j = 0; j < JB; j++) {
      const unsigned d = kk == 0 ? wc[j].x : kk == 1 ? wc[j].y : kk == 2 ? wc[j].z : wc[j].w;
      if (!kNv) {
        const float scale = e8m0_as_scale(sc[j] & 0xFFu);
        bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0);
        bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1);
        bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2);
        bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3);
        wf[j] = (bf16x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      } else {
        const float sb = kk < 2 ? e4m3_value_b<0>(sc[j]) : e4m3_value_b<1>(sc[j]);
        auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
        auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
        auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
        auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
        wf[j] = (bf16x8){(__bf16)(p0[0] * sb), (__bf16)(p0[1] * sb), (__bf16)(p1[0] * sb), (__bf16)(p1[1] * sb),
                         (__bf16)(p2[0] * sb), (__bf16)(p2[1] * sb), (__bf16)(p3[0] * sb), (__bf16)(p3[1] * sb)};
      }
    }
  };
  auto read_x = [&](const uint8_t* xb, int kk, bf16x8 xf[IA]) {
    const int unit16 = ((4 * half + kk) ^ swz) << 4;
#pragma unroll
    for (int i = 0; i < IA; i++) xf[i] = *(const bf16x8*)(xb + laneX + i * 32 * 128 + unit16);
  };
  // Software pipeline inside a stage (fixed by scheduling fences): the
  // activation fragments of step kk+1 are read and the weight operands of
  // step kk+1 are expanded while the 16 MFMAs of step kk run.
  auto compute = [&](auto slot_tag, const unsigned sc[JB]) {
    const uint8_t* xb = g_slot<decltype(slot_tag)::value>().x;
    const uint8_t* wb = g_slot<decltype(slot_tag)::value>().w;
    u32x4 wc[JB];
#pragma unroll
    for (int j = 0; j < JB; j++) wc[j] = *(const u32x4*)(wb + laneW + j * 32 * 32);
    bf16x8 xf[2][IA], wf[2][JB];
    read_x(xb, 0, xf[0]);
    dequant(wc, 0, sc, wf[0]);
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const int c = kk & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (kk < 3) read_x(xb, kk + 1, xf[c ^ 1]);
      if (kk < 3) dequant(wc, kk + 1, sc, wf[c ^ 1]);
#pragma unroll
      for (int i = 0; i < IA; i++)
#pragma unroll
        for (int j = 0; j < JB; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[c][j], xf[c][i], acc[i][j], 0, 0, 0);
      // reads first, then each MFMA followed by a share of the expansion
      // (JB fragments of 8 weights per step, about 16 VALU each for NVFP4
      // and 4-8 for MXFP4, spread over the IA x JB MFMAs)
      constexpr int kVpm = IA == 4 ? (kNv ? 4 : 2) : (kNv ? 2 : 1);
      __builtin_amdgcn_sched_group_barrier(0x100, IA, 0);
#pragma unroll
      for (int g = 0; g < IA * JB; g++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kVpm, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // one stage s in ring slot B: fetch the next stage's scales, wait for
  // stage s (stage s+1's CJX + CJW copies and the JB scale loads may stay
  // in flight; NVFP4's two-byte scale loads only make the wait longer), meet, refill the slot of stage s-1 with stage s+2 (clamped to
  // the last stage near the end: the copy lands in a free slot), multiply.
  // Slot indices are compile-time constants (the loop is unrolled by 3).
  unsigned sc_cur[JB], sc_nxt[JB];
  // (scheduling fences keep the scale loads and the copies where they are
  // written: the scheduler would sink them next to their first use)
  auto step = [&](auto slot_tag, int s) {
    constexpr int B = decltype(slot_tag)::value;
    __builtin_amdgcn_sched_barrier(0);
    load_scales(min(s + 1, nstages - 1), sc_nxt);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<CJX + CJW + JB>();
    __builtin_amdgcn_s_barrier();  // no fence: the prefetched stages stay in flight
    __builtin_amdgcn_sched_barrier(0);
    issue(std::integral_constant<int, (B + kGRing - 1) % kGRing>{}, min(s + kGRing - 1, nstages - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(slot_tag, sc_cur);
#pragma unroll
    for (int j = 0; j < JB; j++) sc_cur[j] = sc_nxt[j];
  };
  static_assert(kGRing == 3, "the stage loop is unrolled by the ring depth");
  // prologue: stages 0, 1 in flight
  issue(std::integral_constant<int, 0>{}, 0);
  issue(std::integral_constant<int, 1>{}, min(1, nstages - 1));
  load_scales(0, sc_cur);
  // whole trips of three stages (no branch inside a trip), then up to two
  int s = 0;
  for (; s + 3 <= nstages; s += 3) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
    step(std::integral_constant<int, 2>{}, s + 2);
  }
  if (s < nstages) step(std::integral_constant<int, 0>{}, s);
  if (s + 1 < nstages) step(std::integral_constant<int, 1>{}, s + 1);
  wait_vmcnt<0>();

  const float st = kNv ? *gscale : 1.0f;
  if constexpr (kBf16Out) {
    // lane (r32, half) holds, for each q, output columns 8q + 4 half + 0..3
    // of its row; lanes l and l ^ 32 swap halves so that each stores whole
    // 16-byte units (8 columns): half 0 the units q = 0, 1, half 1 the units
    // q = 2, 3 (partial 8-byte stores wrote about 1.4x the output bytes)
#pragma unroll
    for (int i = 0; i < IA; i++) {
      const int64_t row = m0 + wm * WROWS + i * 32 + r32;
#pragma unroll
      for (int j = 0; j < JB; j++) {
        u32x2 pk[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; e++) v[e] = kNv ? acc[i][j][4 * q + e] * st : acc[i][j][4 * q + e];
          pk[q] = (u32x2){f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16),
                          f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16)};
        }
#pragma unroll
        for (int a = 0; a < 2; a++) {
          const u32x2 keep = half ? pk[2 + a] : pk[a];  // unit q = 2 half + a, own 4 columns
          const u32x2 send = half ? pk[a] : pk[2 + a];  // what the partner needs
          const u32x2 got = {(unsigned)__shfl_xor((int)send.x, 32, 64), (unsigned)__shfl_xor((int)send.y, 32, 64)};
          const u32x4 unit = half ? (u32x4){got.x, got.y, keep.x, keep.y} : (u32x4){keep.x, keep.y, got.x, got.y};
          const int64_t col = n0 + wn * WCOLS + j * 32 + 8 * (2 * half + a);
          if (row >= m || col >= n) continue;
          uint16_t* dst = (uint16_t*)y + row * n + col;
          if (col + 8 <= n && (n & 7) == 0) {
            *(u32x4*)dst = unit;
          } else {
            const unsigned w[4] = {unit.x, unit.y, unit.z, unit.w};
            for (int e = 0; e < 8 && col + e < n; e++) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < IA; i++) {
    const int64_t row = m0 + wm * WROWS + i * 32 + r32;
    if (row >= m) continue;
#pragma unroll
    for (int j = 0; j < JB; j++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int64_t col = n0 + wn * WCOLS + j * 32 + q * 8 + 4 * half;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] = kNv ? acc[i][j][4 * q + e] * st : acc[i][j][4 * q + e];
        if (col + 3 < n) {
          if (kBf16Out) {
            u32x2 o = {f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16),
                       f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16)};
            *(u32x2*)((uint16_t*)y + row * n + col) = o;
          } else {
            *(f32x4*)((float*)y + row * n + col) = (f32x4){v[0], v[1], v[2], v[3]};
          }
        } else {
          for (int e = 0; e < 4 && col + e < n; e++) {
            if (kBf16Out)
              ((uint16_t*)y)[row * n + col + e] = f32_to_bf16_rne(v[e]);
            else
              ((float*)y)[row * n + col + e] = v[e];
          }
        }
      }
    }
  }
}

#ifndef MXQ_W4A16_GEMM_WAVES
#define MXQ_W4A16_GEMM_WAVES 8
#endif
constexpr int kGemmWaves = MXQ_W4A16_GEMM_WAVES;
// wave-grid rows: MXFP4 2 (2 x 4), NVFP4 1 (1 x 8)
#ifndef MXQ_GEMM_WNR_MX
#define MXQ_GEMM_WNR_MX 2
#endif
#ifndef MXQ_GEMM_WNR_NV
#define MXQ_GEMM_WNR_NV 1
#endif

template <bool kNv>
static void launch_gemm(const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n, int64_t k,
                        const void* x, int64_t m, void* y, bool bf16_out, hipStream_t st) {
  constexpr int WNR = kGemmWaves == 4 ? 2 : (kNv ? MXQ_GEMM_WNR_NV : MXQ_GEMM_WNR_MX);
  const unsigned tiles = (unsigned)(((m + kGBM - 1) / kGBM) * ((n + kGBN - 1) / kGBN));
  if (bf16_out)
    hipLaunchKernelGGL((k_w4a16_gemm<kNv, true, kGemmWaves, WNR>), dim3(tiles), dim3(64 * kGemmWaves), 0, st, wq,
                       ws, gscale, n, k, (const uint16_t*)x, m, y);
  else
    hipLaunchKernelGGL((k_w4a16_gemm<kNv, false, kGemmWaves, WNR>), dim3(tiles), dim3(64 * kGemmWaves), 0, st, wq,
                       ws, gscale, n, k, (const uint16_t*)x, m, y);
}

template <bool kNv, int R, int U, int W>
static void launch_decode(const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n, int64_t k,
                          const void* x, int64_t m, void* y, bool bf16_out, hipStream_t st) {
  dim3 grid((unsigned)((n + 16 * R - 1) / (16 * R)), (unsigned)((m + 15) / 16));
  if (bf16_out)
    hipLaunchKernelGGL((k_w4a16_decode<kNv, R, U, W, true>), grid, dim3(64 * W), 0, st, wq, ws, gscale, n, k,
                       (const uint16_t*)x, m, y);
  else
    hipLaunchKernelGGL((k_w4a16_decode<kNv, R, U, W, false>), grid, dim3(64 * W), 0, st, wq, ws, gscale, n, k,
                       (const uint16_t*)x, m, y);
}

// ---------------------------------------------------------------------------
// Decode kernel for m <= 16, k % 512 == 0 (MXFP4): the weight stream is
// moved by direct buffer -> LDS copies, so the bytes in flight are bounded by
// LDS, not by staging registers, and the arithmetic is the 16x16x32 bf16
// MFMA (its cost does not grow with m; rows m..15 of the activation operand
// read a shared zero row).
//   * A block is NW waves; wave w owns weight rows n0 + 16w .. +16 for the
//     whole of k.  k advances in stages of 512 (256 code bytes and 16 scale
//     bytes per row, 1 KiB of activations per activation row) through a ring
//     of NR LDS stages.
//   * Every wave loads its own rows' codes (4 x 1 KiB, four 256-B row
//     segments per instruction) and scales (16 rows x 16 B of E8M0, one
//     4-byte-per-lane instruction; NVFP4: 16 rows x 32 B of E4M3, two), and
//     its share of the activation rows (one 1 KiB
//     instruction per row; every wave issues the same number, surplus ones
//     fill a scratch row, so the wait counts are compile-time constants).
//   * LDS swizzles (applied on the global side of the copy): code unit u of
//     row r sits at slot u ^ (r & 15); activation unit u of row i at
//     u ^ (i & 15).  The 16 lanes of a fragment read touch 16 distinct bank
//     groups.
//   * Fragments: lane (col = l % 16, g = l / 16) takes code unit 4i + g of
//     its weight row (32 k = one MXFP4 block or two NVFP4 blocks, i =
//     0..3), expands it to four exact bf16x8 operands (dequant_chunk), and
//     pairs operand j with
//     activation unit 16i + 4g + j of activation row col (the MFMA k slots
//     are a permutation of the stage's k, the same on both sides).
//   * One s_barrier per stage (after the wave's own copies of stage s have
//     landed) makes the other waves' activation copies visible and frees the
//     ring slot for the copy of stage s + NR - 1.
//   * Blocks start their k loop at staggered stages: block b walks the
//     stages from (b / 8) mod nst on, so the blocks resident at one time
//     (dispatched round robin over the eight XCDs) read rows at different
//     column offsets instead of all at the same one (about 10 % faster on
//     a 28672 x 8192 weight).  The k order of a block's sum changes with
//     its rotation; the result is still one fixed order per output row.
//   * NVFP4: the tensor scale multiplies the fp32 sums in the epilogue.
// Short waves skip their padding activation copy (1) or re-read activation
// rows into a scratch row so every wave issues the same count (0).
// Interleaved A/B on 28672 x 8192, bitwise-equal results: m = 4 22.2-22.3
// against 22.8-23.2 us, m = 16 24.0-24.1 against 25.1-26.0, m = 64
// 51.8-52.4 against 55.8-56.2, NVFP4 m = 16 33.0 against 33.5.
#ifndef MXQ_DD_XNEED
#define MXQ_DD_XNEED 1
#endif
#ifndef MXQ_DD_XSKIP
#define MXQ_DD_XSKIP 1
#endif
// The wave index in a scalar register (1: readfirstlane) or as a vector
// value (0).  Interleaved A/B: m = 16 23.8-24.1 against 24.0-24.9 us, m = 64
// 51.0-51.2 against 51.9-52.2, NVFP4 m = 16 32.1 against 32.6, m = 4 even.
#ifndef MXQ_DD_WUNI
#define MXQ_DD_WUNI 1
#endif
// NVFP4 with up to 4 activation rows: E4M3 block scales applied to the
// 16-k sums of 4x4x4 block MFMAs (1) or to every weight element before the
// 16x16x32 MFMA (0).
#ifndef MXQ_DD_NVB
#define MXQ_DD_NVB 1
#endif
// NVFP4 with 5..8 activation rows and resident scales: the 4x4x4 form on two
// row quads (256-k stages, 4 slots) (1), or the 16-row ring (0).
#ifndef MXQ_DD_NVB8
#define MXQ_DD_NVB8 1
#endif
// The same 4x4x4 form for MXFP4 at up to 4 activation rows (1), or the
// 16x16x32 MFMA with 12 zero activation rows (0).
#ifndef MXQ_DD_MXB
#define MXQ_DD_MXB 0
#endif
// Longest k whose scale rows the decode ring can keep resident in LDS.
constexpr int kDdResK = 8192;
// Stage geometry of the decode ring for KS k per stage (512 or 256).
template <int KS, bool kNv>
struct DdGeom {
  static constexpr int RowB = KS / 2;                 // code bytes per weight row
  static constexpr int U = RowB / 16;                 // 16-byte units per weight row (16 or 8)
  static constexpr int RPI = 64 / U;                  // weight rows per 1-KiB copy (4 or 8)
  static constexpr int WC = 16 / RPI;                 // weight copies per wave (16 rows)
  static constexpr int XRowB = 2 * KS;                // bf16 activation bytes per row
  static constexpr int XRPI = 1024 / XRowB;           // activation rows per 1-KiB copy (1 or 2)
  static constexpr int ScB = kNv ? KS / 16 : KS / 32;  // scale bytes per weight row (8 .. 32)
  // scales sit in 256-byte pieces, 16 bytes per row per piece; a row with 8
  // scale bytes fills the first half of its 16 (the copy repeats them)
  static constexpr int SCP = ScB > 16 ? ScB / 16 : 1;  // scale pieces (copies) per wave
  static constexpr int SPL = ScB < 16 ? ScB / 4 : 4;   // distinct 4-byte parts per row and piece
  static constexpr int STEPS = KS / 128;              // 128-k chunks (4 per lane group) per stage
};

// One ring slot: codes, activations and scales of one stage.  Every slot is
// its own LDS variable and every slot index below is a compile-time
// constant, so the compiler can tell that the reads of slot b do not touch
// the slots whose copies are still in flight (one shared array would make it
// wait for every outstanding copy before the first read).
template <int MT, int NW, int KS, bool kNv, bool RS>
struct DdSlot {
  using G = DdGeom<KS, kNv>;
  uint8_t w[16 * NW * G::RowB];
  uint8_t x[(MT + 1 + G::XRPI) * G::XRowB];  // MT activation rows, a zero row, scratch rows
  uint8_t s[RS ? 16 : NW * G::SCP * 256];    // stage scales (resident scales: unused)
};
// (16-byte alignment for the resident-scale rings, whose LDS is full to the
// last KiB with NVFP4 scales: a uniform shift of a slot keeps its bank
// pattern)
template <int MT, int NW, int KS, bool kNv, bool RS, int B>
__device__ __forceinline__ DdSlot<MT, NW, KS, kNv, RS>& dd_slot() {
  __shared__ __attribute__((aligned(RS ? 16 : 1024))) DdSlot<MT, NW, KS, kNv, RS> slot;
  return slot;
}

template <bool kNv, int MT, int NW, int NR, int KS, bool RS, bool kBf16Out>
__global__ __launch_bounds__(64 * NW, 1) void k_w4a16_decode_dma(const uint8_t* __restrict__ wq,
                                                                const uint8_t* __restrict__ ws,
                                                                const float* __restrict__ gscale, int64_t n,
                                                                int64_t k, const uint16_t* __restrict__ x,
                                                                int64_t m, void* __restrict__ y) {
  using G = DdGeom<KS, kNv>;
  using Slot = DdSlot<MT, NW, KS, kNv, RS>;
  constexpr int RB = 16 * NW;                          // weight rows per block
  constexpr int MTT = (MT + 15) / 16;                  // 16-row activation tiles
  constexpr int XPW = (MT / G::XRPI + NW - 1) / NW;    // activation copies per wave per stage, at most
  constexpr int XC = MT / G::XRPI;                     // activation copies per stage (real rows)
  constexpr int D = G::WC + (RS ? 0 : G::SCP) + XPW;   // copies per wave per stage, at most
  static_assert((MT % 16 == 0 || MT < 16) && NR >= 2 && NR <= 8 && (NR - 2) * D < 64, "tile / ring depth / vmcnt range");
  // the wave index is uniform: held in a scalar register, so the branches
  // on it (xfull) are scalar and its address terms stay off the VGPRs
  const int tid = threadIdx.x, lane = tid & 63, wave = MXQ_DD_WUNI ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  // Activation copies are dealt round robin (copy a to wave a mod NW), so a
  // wave issues XPW or XPW - 1 of them.  With MXQ_DD_XSKIP the short waves
  // issue one copy fewer and wait on their own count (a wave-uniform branch
  // picks the immediate); without it they pad with a re-read of activation
  // rows into a scratch row.
  // Where a wave issues at most one activation copy per stage, the copies of
  // rows at or past m are skipped as well (those rows read the zero row):
  // at m = 1, one copy per stage instead of MT / XRPI.
  const int xc_need = XPW == 1 && MXQ_DD_XNEED ? (int)min((int64_t)XC, (m + G::XRPI - 1) / G::XRPI) : XC;
  const bool xfull = !MXQ_DD_XSKIP || wave + NW * (XPW - 1) < xc_need;
  const int64_t n0 = (int64_t)blockIdx.x * RB;
  const int rows_w = (int)min((int64_t)RB, n - n0);
  const int64_t kq = k / 2, ks = kNv ? k / 16 : k / 32, kx = k * 2;
  const int nst = (int)(k / KS);
  // staggered start, counted in 512-k chunks (the same k order for either
  // stage length)
  const int rot = (int)((blockIdx.x / 8) % (unsigned)(k / 512)) * (512 / KS);
  // absolute stage of loop stage s (a stage past the end is clamped to the last)
  auto stage_of = [&](int s) -> unsigned {
    const int sl0 = min(s, nst - 1);
    return (unsigned)(sl0 + rot < nst ? sl0 + rot : sl0 + rot - nst);
  };
  // Resident scales (k <= kDdResK): the wave's 16 rows x ks scale bytes sit
  // in LDS for the whole k loop, rows padded by 16 B (the 16 rows a fragment
  // read touches then fall in distinct bank groups), instead of per-stage
  // copies of one 8-, 16- or 32-byte request per row and stage.  They make
  // the shorter 256-k stages pay at m = 16 (launch_decode_ring has the
  // figures).
  constexpr int KSMAX = kNv ? kDdResK / 16 : kDdResK / 32;  // scale bytes per row, at most
  constexpr int PU = KSMAX / 64;                            // 16-byte units per lane, at most
  __shared__ __attribute__((aligned(16))) uint8_t sres[RS ? NW * 16 * (KSMAX + 16) : 16];
  const int rsp = (int)ks + 16;                             // LDS pitch of a scale row
  const int upr = (int)(ks >> 4);                           // 16-byte units per scale row

  // zero row (activation rows m..MT-1 of the MFMA operand read it)
  for (int i = tid; i < G::XRowB / 16; i += 64 * NW) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    *(u32x4*)(dd_slot<MT, NW, KS, kNv, RS, 0>().x + MT * G::XRowB + 16 * i) = z;
    if constexpr (NR > 1) *(u32x4*)(dd_slot<MT, NW, KS, kNv, RS, 1>().x + MT * G::XRowB + 16 * i) = z;
    if constexpr (NR > 2) *(u32x4*)(dd_slot<MT, NW, KS, kNv, RS, 2>().x + MT * G::XRowB + 16 * i) = z;
    if constexpr (NR > 3) *(u32x4*)(dd_slot<MT, NW, KS, kNv, RS, 3>().x + MT * G::XRowB + 16 * i) = z;
    if constexpr (NR > 4) *(u32x4*)(dd_slot<MT, NW, KS, kNv, RS, 4>().x + MT * G::XRowB + 16 * i) = z;
    if constexpr (NR > 5) *(u32x4*)(dd_slot<MT, NW, KS, kNv, RS, 5>().x + MT * G::XRowB + 16 * i) = z;
    if constexpr (NR > 6) *(u32x4*)(dd_slot<MT, NW, KS, kNv, RS, 6>().x + MT * G::XRowB + 16 * i) = z;
    if constexpr (NR > 7) *(u32x4*)(dd_slot<MT, NW, KS, kNv, RS, 7>().x + MT * G::XRowB + 16 * i) = z;
  }
  __syncthreads();

  // Copies of stage s into ring slot B.  A stage past the end is clamped to
  // the last one (a re-read from L2 into a slot nobody reads), so every step
  // issues the same copies and waits for the same count, and the code
  // between the copies and the reads has no branch.  Lane offsets are fixed
  // for the whole k loop; a stage only moves the uniform offset.
  unsigned offw[G::WC], offx[XPW];
  int xdst[XPW];
#pragma unroll
  for (int q = 0; q < G::WC; q++) {
    const int row = 16 * wave + G::RPI * q + lane / G::U;  // block row of this lane
    const unsigned unit = (unsigned)((lane % G::U) ^ (row % G::U));
    offw[q] = (unsigned)min(row, rows_w - 1) * (unsigned)kq + (unit << 4);
  }
  // scale copy h: lane i takes row i / 4 of the wave, 4 bytes at 16 h +
  // 4 ((i % 4) % SPL) of the row's stage bytes
  const unsigned offs = (unsigned)min(16 * wave + (lane >> 2), rows_w - 1) * (unsigned)ks +
                        4u * (unsigned)((lane & 3) % G::SPL);
#pragma unroll
  for (int j = 0; j < XPW; j++) {
    const int a = wave + NW * j;  // copy slot (wave-uniform): activation rows XRPI a ..
    const int xr = G::XRPI * a + lane / (64 / G::XRPI);
    const bool real = G::XRPI * a < MT;
    const unsigned unit = (unsigned)((lane % (64 / G::XRPI)) ^ (xr & 15));
    offx[j] = (unsigned)min((int64_t)xr, m - 1) * (unsigned)kx + (unit << 4);
    xdst[j] = (real ? G::XRPI * a : MT + 1) * G::XRowB;
  }
  // buffer resources over the block's weight, scale and activation panels
  // (32-bit lane offsets; the panels stay below 2^31 bytes for k <= 2^24)
  const __amdgpu_buffer_rsrc_t rw = panel_rsrc(wq + n0 * kq, rows_w * kq);
  const __amdgpu_buffer_rsrc_t rs = panel_rsrc(ws + n0 * ks, rows_w * ks);
  const __amdgpu_buffer_rsrc_t rx = panel_rsrc(x, m * kx);
  auto issue = [&](auto slot_tag, int s) {
    constexpr int B = decltype(slot_tag)::value;
    Slot& sl = dd_slot<MT, NW, KS, kNv, RS, B>();
    const unsigned sc = stage_of(s);
    // activation copies first: their L2 round trip then overlaps the weight
    // copies' longer one (a copy-only probe of the m = 4 ring: 22.0 against
    // 22.7 us with them last; the kernel itself gains about 1 %)
#pragma unroll
    for (int j = 0; j < XPW; j++)
      if (j < XPW - 1 || xfull) bdma16(rx, offx[j], sc * G::XRowB, sl.x + xdst[j]);
#pragma unroll
    for (int q = 0; q < G::WC; q++)
      bdma16_nt(rw, offw[q], sc * G::RowB, sl.w + (16 * wave + G::RPI * q) * G::RowB);
    // LDS: piece h of the wave's rows at s + (SCP wave + h) * 256, row r of
    // the wave at + 16 r
    if constexpr (!RS) {
#pragma unroll
      for (int h = 0; h < G::SCP; h++) bdma4(rs, offs + 16u * h, sc * G::ScB, sl.s + (G::SCP * wave + h) * 256);
    }
  };

  // Up to 4 (MXFP4) or 8 (NVFP4) activation rows: 4x4x4 block MFMAs
  // (acc[q] holds activation rows 4q..4q+3 of the lane's weight row, over
  // its lane group's chunks); otherwise 16x16x32 MFMAs on pre-scaled
  // weights
  constexpr bool kB4 = kNv ? (MT == 4 || MT == 8) && MXQ_DD_NVB : MT == 4 && MXQ_DD_MXB;
  constexpr int NQ = MT / 4;  // activation row quads of the 4x4x4 form
  constexpr int NACC = kB4 ? NQ : MTT;
  f32x4 acc[NACC];
#pragma unroll
  for (int t = 0; t < NACC; t++) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int wrow = 16 * wave + col;  // this lane's block weight row
  auto compute = [&](auto slot_tag, unsigned sc) {
    constexpr int B = decltype(slot_tag)::value;
    const Slot& sl = dd_slot<MT, NW, KS, kNv, RS, B>();
    // this lane's row's scale bytes of the stage (absolute stage sc): ScB
    // (E8M0 per 32 k or E4M3 per 16), word w = bytes 4w .. 4w+3
    unsigned svs[G::SCP * 4];
    const uint8_t* sp = sres + (16 * wave + col) * rsp + sc * G::ScB;
    if constexpr (RS && kNv) {
      // read per chunk below: the two bytes of lane group g's chunk sit at a
      // lane-dependent offset, and one 2-byte LDS read replaces selecting
      // them out of the stage's words
    } else if constexpr (RS) {
      if constexpr (G::ScB >= 16) {
#pragma unroll
        for (int h = 0; h < G::SCP; h++) {
          const u32x4 sv = *(const u32x4*)(sp + 16 * h);
          svs[4 * h] = sv.x; svs[4 * h + 1] = sv.y; svs[4 * h + 2] = sv.z; svs[4 * h + 3] = sv.w;
        }
      } else {
        const u32x2 sv = *(const u32x2*)sp;
        svs[0] = sv.x; svs[1] = sv.y; svs[2] = 0u; svs[3] = 0u;
      }
    } else {
#pragma unroll
      for (int h = 0; h < G::SCP; h++) {
        const u32x4 sv = *(const u32x4*)(sl.s + (G::SCP * wave + h) * 256 + 16 * col);
        svs[4 * h] = sv.x; svs[4 * h + 1] = sv.y; svs[4 * h + 2] = sv.z; svs[4 * h + 3] = sv.w;
      }
    }
    if constexpr (kB4) {
      // Up to 4 (MXFP4) or 8 (NVFP4) activation rows, in quads of 4: 4x4x4
      // block MFMAs.  Lane (col, g) is MFMA block 4g + col / 4, column
      // col % 4: its weight row's 32 k of chunk 4i + g in bf16 (exact),
      // against activation row 4q + col % 4 at the same k for quad q, so
      // the lane's D column is its own weight row.  MXFP4: the E8M0
      // scale rides in the convert.  NVFP4: the codes are converted
      // unscaled and each 16-k block's sum takes its row's E4M3 scale in 4
      // FMAs (instead of a multiply per weight element).
      const uint8_t* xb[NQ];
      int xsw[NQ];
#pragma unroll
      for (int q = 0; q < NQ; q++) {
        const int xr = 4 * q + (col & 3);
        xb[q] = sl.x + (xr < m ? xr : MT) * G::XRowB;
        xsw[q] = xr < m ? (xr & 15) : 0;
      }
#pragma unroll
      for (int i = 0; i < G::STEPS; i++) {
        const u32x4 cw = *(const u32x4*)(sl.w + wrow * G::RowB + (((4 * i + g) ^ (col % G::U)) << 4));
        unsigned sb2;
        if constexpr (kNv && RS)
          sb2 = *(const uint16_t*)(sp + 8 * i + 2 * g);
        else if constexpr (kNv)
          sb2 = (svs[2 * i + (g >> 1)] >> (16 * (g & 1))) & 0xFFFFu;
        else
          sb2 = (svs[i] >> (8 * g)) & 0xFFu;
        const float cs = kNv ? 1.0f : e8m0_as_scale(sb2);
        const unsigned d[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int h = 0; h < 2; h++) {  // the chunk's two 16-k halves (NVFP4 blocks)
          f32x4 db[NQ];
#pragma unroll
          for (int q = 0; q < NQ; q++) db[q] = kNv ? (f32x4){0.f, 0.f, 0.f, 0.f} : acc[q];
#pragma unroll
          for (int jj = 0; jj < 2; jj++) {
            const int j = 2 * h + jj;  // k 8j .. 8j + 7 of the chunk
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], cs, 0);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], cs, 1);
            const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], cs, 2);
            const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], cs, 3);
#pragma unroll
            for (int q = 0; q < NQ; q++) {
              const bf16x8 xa = *(const bf16x8*)(xb[q] + ((16 * i + ((4 * g + j) ^ xsw[q])) << 4));
              db[q] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k((bf16x4){xa[0], xa[1], xa[2], xa[3]},
                                                             (bf16x4){p0[0], p0[1], p1[0], p1[1]}, db[q], 0, 0, 0);
              db[q] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k((bf16x4){xa[4], xa[5], xa[6], xa[7]},
                                                             (bf16x4){p2[0], p2[1], p3[0], p3[1]}, db[q], 0, 0, 0);
            }
          }
          if constexpr (kNv) {
            const float sbk = h ? e4m3_value_b<1>(sb2) : e4m3_value_b<0>(sb2);
#pragma unroll
            for (int q = 0; q < NQ; q++)
#pragma unroll
              for (int e = 0; e < 4; e++) acc[q][e] = __builtin_fmaf(sbk, db[q][e], acc[q][e]);
          } else {
#pragma unroll
            for (int q = 0; q < NQ; q++) acc[q] = db[q];
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < G::STEPS; i++) {
      const u32x4 cw = *(const u32x4*)(sl.w + wrow * G::RowB + (((4 * i + g) ^ (col % G::U)) << 4));
      bf16x8 wf[4];
      if constexpr (kNv && RS) {
        // the two E4M3 scales of chunk 4i + g: bytes 8i + 2g, 8i + 2g + 1
        dequant_chunk<true>(cw, *(const uint16_t*)(sp + 8 * i + 2 * g), wf);
      } else if constexpr (kNv) {
        dequant_chunk<true>(cw, (svs[2 * i + (g >> 1)] >> (16 * (g & 1))) & 0xFFFFu, wf);
      } else {
        dequant_chunk<false>(cw, (svs[i] >> (8 * g)) & 0xFFu, wf);
      }
#pragma unroll
      for (int t = 0; t < MTT; t++) {
        const int xr = 16 * t + col;
        const bool xreal = xr < m;
        const uint8_t* xb = sl.x + (xreal ? xr : MT) * G::XRowB;
        const int xsw = xreal ? (xr & 15) : 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const bf16x8 xa = *(const bf16x8*)(xb + ((16 * i + ((4 * g + j) ^ xsw)) << 4));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wf[j], acc[t], 0, 0, 0);
        }
      }
    }
  };

  // one stage: wait for its copies (NR - 2 later stages may stay in
  // flight), meet the other waves, refill the slot everyone finished in the
  // previous stage, multiply.  Every step issues, so the count is constant
  // and the code between the copies and the reads has no branch.
  auto step = [&](auto slot_tag, int s) {
    constexpr int B = decltype(slot_tag)::value;
    // this wave's copies of stage s have landed and its reads of the slot
    // about to be refilled are complete (lgkmcnt(0)), then the barrier
    constexpr int N = (NR - 2) * D, N1 = (NR - 2) * (D - 1);
    if (xfull)
      __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    else
      __builtin_amdgcn_s_waitcnt((N1 & 15) | ((N1 >> 4) << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    issue(std::integral_constant<int, (B + NR - 1) % NR>{}, s + NR - 1);
    if (s < nst) compute(slot_tag, stage_of(s));
  };

  // prologue: stages 0 .. NR-2 in flight, then stage 0.  The loop below
  // starts at the step that refills slot 0, so that the copies of one trip
  // target the slots in the same order as the prologue's.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1 % NR>;
  using I2 = std::integral_constant<int, 2 % NR>;
  using I3 = std::integral_constant<int, 3 % NR>;
  using I4 = std::integral_constant<int, 4 % NR>;
  using I5 = std::integral_constant<int, 5 % NR>;
  using I6 = std::integral_constant<int, 6 % NR>;
  using I7 = std::integral_constant<int, 7 % NR>;
  // resident scales: PU 16-byte loads per lane (unit i = lane + 64 p of the
  // wave's 16 x ks bytes; units past the wave's rows re-read a valid unit
  // and are dropped), issued before the ring's first copies
  u32x4 rsv[RS ? PU : 1];
  if constexpr (RS) {
#pragma unroll
    for (int p = 0; p < PU; p++) {
      const int i = lane + 64 * p;
      const int r = i / upr, c = i - r * upr;
      const int row = min(16 * wave + min(r, 15), rows_w - 1);
      rsv[p] = *(const u32x4*)(ws + (n0 + row) * ks + 16 * c);
    }
  }
  issue(I0{}, 0);
  if constexpr (NR > 2) issue(I1{}, 1);
  if constexpr (NR > 3) issue(I2{}, 2);
  if constexpr (NR > 4) issue(I3{}, 3);
  if constexpr (NR > 5) issue(I4{}, 4);
  if constexpr (NR > 6) issue(I5{}, 5);
  if constexpr (NR > 7) issue(I6{}, 6);
  if constexpr (RS) {
    // the scale loads are older than the NR - 1 stages of copies in flight;
    // only this wave reads its rows' scales, so no barrier is needed
    if (xfull)
      wait_vmcnt<(NR - 1) * D>();
    else
      wait_vmcnt<(NR - 1) * (D - 1)>();
#pragma unroll
    for (int p = 0; p < PU; p++) {
      const int i = lane + 64 * p;
      const int r = i / upr, c = i - r * upr;
      if (r < 16) *(u32x4*)(sres + (16 * wave + r) * rsp + 16 * c) = rsv[p];
    }
  }
  step(I0{}, 0);
  for (int s = 1; s < nst; s += NR) {
    step(I1{}, s);
    if constexpr (NR > 2) step(I2{}, s + 1);
    if constexpr (NR > 3) step(I3{}, s + 2);
    if constexpr (NR > 4) step(I4{}, s + 3);
    if constexpr (NR > 5) step(I5{}, s + 4);
    if constexpr (NR > 6) step(I6{}, s + 5);
    if constexpr (NR > 7) step(I7{}, s + 6);
    step(I0{}, s + NR - 1);
  }
  wait_vmcnt<0>();

  const float st = kNv ? *gscale : 1.0f;
  const int64_t nn = n0 + wrow;
  if constexpr (kB4) {
    // sum the four lane groups' k shares (the same order in every lane),
    // then lane group g writes activation rows 4q + g
#pragma unroll
    for (int q = 0; q < NQ; q++) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        acc[q][e] += __shfl_xor(acc[q][e], 16);
        acc[q][e] += __shfl_xor(acc[q][e], 32);
      }
      const float v = g == 0 ? acc[q][0] : g == 1 ? acc[q][1] : g == 2 ? acc[q][2] : acc[q][3];
      const int64_t mm = 4 * q + g;
      if (nn < n && mm < m) {
        const float o = v * st;
        if (kBf16Out)
          ((uint16_t*)y)[mm * n + nn] = f32_to_bf16_rne(o);
        else
          ((float*)y)[mm * n + nn] = o;
      }
    }
    return;
  }
  // lane holds y[16t + 4g + i][n0 + wrow]
  if (nn < n) {
#pragma unroll
    for (int t = 0; t < MTT; t++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t mm = 16 * t + 4 * g + i;
        if (mm >= m) continue;
        const float o = kNv ? acc[t][i] * st : acc[t][i];
        if (kBf16Out)
          ((uint16_t*)y)[mm * n + nn] = f32_to_bf16_rne(o);
        else
          ((float*)y)[mm * n + nn] = o;
      }
  }
}

template <bool kNv, int MT, int NW, int NR, int KS, bool RS = false>
static void launch_decode_dma(const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n, int64_t k,
                              const void* x, int64_t m, void* y, bool bf16_out, hipStream_t st) {
  const dim3 grid((unsigned)((n + 16 * NW - 1) / (16 * NW)));
  if (bf16_out)
    hipLaunchKernelGGL((k_w4a16_decode_dma<kNv, MT, NW, NR, KS, RS, true>), grid, dim3(64 * NW), 0, st, wq, ws,
                       gscale, n, k, (const uint16_t*)x, m, y);
  else
    hipLaunchKernelGGL((k_w4a16_decode_dma<kNv, MT, NW, NR, KS, RS, false>), grid, dim3(64 * NW), 0, st, wq, ws,
                       gscale, n, k, (const uint16_t*)x, m, y);
}

// Decode ring configurations <MT, NW, NR, KS> by activation rows.
#ifndef MXQ_DD_KS4
#define MXQ_DD_KS4 512
#define MXQ_DD_NR4 3
#endif
#ifndef MXQ_DD_KS16
#define MXQ_DD_KS16 512
#define MXQ_DD_NR16 3
#endif
// Stage-scale rings (k > kDdResK).  NVFP4 at 5..16 rows: 256-k stages in a
// 5-slot ring, about 4 % faster than the MXFP4 shape (measured on 28672 x
// 8192, m = 16: 41.0 vs 42.6 us); for MXFP4 the shorter stages' scale
// copies cost more (30.1 vs 26.6 us)
#ifndef MXQ_DD_KS16_NV
#define MXQ_DD_KS16_NV 256
#define MXQ_DD_NR16_NV 5
#endif
#ifndef MXQ_DD_KS32
#define MXQ_DD_KS32 256
#define MXQ_DD_NR32 4
#endif
// Resident-scale rings (k <= kDdResK) for up to 16 activation rows: up to 4
// rows keep the 512-k, 3-slot ring; 5..16 rows take 256-k stages in a
// 4-slot ring (ring and resident scales fit in LDS).  Measured on 28672 x
// 8192: MXFP4 m = 16 24.7 us against 26.7 us for the 512-k ring with stage
// scale copies and 29.1 us for the same 256-k ring with stage scale copies
// (8 bytes per row and stage); NVFP4 m = 16 39.3 against 40.7 us (5 slots,
// stage copies); m = 4 unchanged (24.2 vs 24.0 us).
#ifndef MXQ_DD_RS
#define MXQ_DD_RS 1
#endif
#ifndef MXQ_DD_RS4
#define MXQ_DD_RS4 3, 512
#endif
#ifndef MXQ_DD_RS16
#define MXQ_DD_RS16 4, 256
#endif
// MXFP4 at m = 1 on a 1-row activation tile with NR 512-k slots (which
// LDS then holds up to 4 of) instead of the 4-row, 3-slot ring (0).
// Interleaved A/B on 28672 x 8192: NR = 3 21.41 against 21.68 us (within
// the run-to-run spread), NR = 4 22.94; not used.
#ifndef MXQ_DD_M1NR
#define MXQ_DD_M1NR 0
#endif
#ifndef MXQ_DD_RS16_NV
#define MXQ_DD_RS16_NV 4, 256
#endif
template <bool kNv>
static void launch_decode_ring(const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n, int64_t k,
                               const void* x, int64_t m, void* y, bool bf16_out, hipStream_t st) {
  const bool res = MXQ_DD_RS && k <= kDdResK;
  if constexpr (!kNv && MXQ_DD_M1NR > 0) {
    if (m == 1 && res) {
      launch_decode_dma<false, 1, 7, MXQ_DD_M1NR, 512, true>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
      return;
    }
  }
  if (m <= 16 && res) {
    if (m <= 4)
      launch_decode_dma<kNv, 4, 7, MXQ_DD_RS4, true>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
    else if (kNv && MXQ_DD_NVB8 && m <= 8)
      launch_decode_dma<kNv, 8, 7, 4, 256, true>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
    else if constexpr (kNv)
      launch_decode_dma<kNv, 16, 7, MXQ_DD_RS16_NV, true>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
    else
      launch_decode_dma<kNv, 16, 7, MXQ_DD_RS16, true>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  } else if (m <= 4)
    launch_decode_dma<kNv, 4, 7, MXQ_DD_NR4, MXQ_DD_KS4>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  else if (m <= 16 && kNv)
    launch_decode_dma<kNv, 16, 7, MXQ_DD_NR16_NV, MXQ_DD_KS16_NV>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  else if (m <= 16)
    launch_decode_dma<kNv, 16, 7, MXQ_DD_NR16, MXQ_DD_KS16>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  else if (m <= 32)
    launch_decode_dma<kNv, 32, 7, MXQ_DD_NR32, MXQ_DD_KS32>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  else if (m <= 48)
    launch_decode_dma<kNv, 48, 7, 3, 256>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  else
    launch_decode_dma<kNv, 64, 7, 3, 256>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
}

// Fewest activation rows that take the decode ring: MXFP4 from 1 (the ring
// measured 21.5-21.7 against 22.6-23.1 us for the vector-ALU kernel at m = 1
// on 28672 x 8192, interleaved A/B, with the activation copies of rows past
// m skipped), NVFP4 from 2 (at m = 1 the vector-ALU kernel, which applies
// each E4M3 scale once per 16 products, measured even with the ring).
#ifndef MXQ_DD_MXMIN
#define MXQ_DD_MXMIN 1
#endif
#ifndef MXQ_DD_NVMIN
#define MXQ_DD_NVMIN 2
#endif
#ifndef MXQ_DD_MAXM
#define MXQ_DD_MAXM 64
#endif

hipError_t launch_w4a16(bool nv, const uint8_t* wq, const uint8_t* ws, const float* gscale, int64_t n,
                        int64_t k, const void* x, int64_t m, void* y, bool bf16_out, hipStream_t st) {
  // The decode ring from m = MXQ_DD_MXMIN (MXFP4) or MXQ_DD_NVMIN (NVFP4)
  // activation rows, for weights of at least 14336 rows and k % 512 == 0.
  const bool ring = k % 512 == 0 && k <= (1 << 24) && n >= 16 * 7 * 128;
  // m = MAXM+1 .. 2 MAXM in two passes, the first over MAXM activation rows
  // on the ring, the second over the rest by this same dispatch: two reads of
  // the weight cost less than the tiled GEMM at these heights (28672 x 8192:
  // about 2 x 60 us against 156 us for the GEMM at m = 128).
  if (ring && m > MXQ_DD_MAXM && m <= 2 * MXQ_DD_MAXM) {
    const hipError_t e = launch_w4a16(nv, wq, ws, gscale, n, k, x, MXQ_DD_MAXM, y, bf16_out, st);
    if (e != hipSuccess) return e;
    return launch_w4a16(nv, wq, ws, gscale, n, k, (const uint16_t*)x + MXQ_DD_MAXM * k, m - MXQ_DD_MAXM,
                        (uint8_t*)y + MXQ_DD_MAXM * n * (bf16_out ? 2 : 4), bf16_out, st);
  }
  if (ring && m >= (nv ? MXQ_DD_NVMIN : MXQ_DD_MXMIN) && m <= MXQ_DD_MAXM) {
    nv ? launch_decode_ring<true>(wq, ws, gscale, n, k, x, m, y, bf16_out, st)
       : launch_decode_ring<false>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  } else if (!nv && m >= 5 && m <= 16) {
    const dim3 grid((unsigned)((n + 63) / 64));
    if (bf16_out)
      hipLaunchKernelGGL(k_w4a16_decode_mfma<true>, grid, dim3(256), 0, st, wq, ws, n, k, (const uint16_t*)x, m, y);
    else
      hipLaunchKernelGGL(k_w4a16_decode_mfma<false>, grid, dim3(256), 0, st, wq, ws, n, k, (const uint16_t*)x, m, y);
  } else if (m <= 4) {
    switch ((int)m) {
      case 1: nv ? launch_decode_valu<true, 1>(wq, ws, gscale, n, k, x, y, bf16_out, st)
                 : launch_decode_valu<false, 1>(wq, ws, gscale, n, k, x, y, bf16_out, st); break;
      case 2: nv ? launch_decode_valu<true, 2>(wq, ws, gscale, n, k, x, y, bf16_out, st)
                 : launch_decode_valu<false, 2>(wq, ws, gscale, n, k, x, y, bf16_out, st); break;
      case 3: nv ? launch_decode_valu<true, 3>(wq, ws, gscale, n, k, x, y, bf16_out, st)
                 : launch_decode_valu<false, 3>(wq, ws, gscale, n, k, x, y, bf16_out, st); break;
      default: nv ? launch_decode_valu<true, 4>(wq, ws, gscale, n, k, x, y, bf16_out, st)
                  : launch_decode_valu<false, 4>(wq, ws, gscale, n, k, x, y, bf16_out, st); break;
    }
  } else if (m >= 128 && k % 64 == 0 && k < (1 << 23)) {
    // the GEMM tile addresses its 256-row activation panel (512 k bytes)
    // with 32-bit buffer offsets: k < 2^23 keeps it below 2^32 bytes;
    // longer rows take the decode kernel (64-bit addressing)
    nv ? launch_gemm<true>(wq, ws, gscale, n, k, x, m, y, bf16_out, st)
       : launch_gemm<false>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  } else if (nv) {
    launch_decode<true, 2, 2, 4>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  } else {
    launch_decode<false, 2, 4, 4>(wq, ws, gscale, n, k, x, m, y, bf16_out, st);
  }
  return hipGetLastError();
}

}  // namespace mxq
