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
#include <type_traits>

#include "mxq_device.h"
#include "mxq_gemm_common.h"
#include "mxq_launch.h"

namespace mxq {


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

// ---------------------------------------------------------------------------
// Ring kernel (k % 1024 == 0).  Block tile 128 (m) x 256 (n) of eight 64 x 64
// wave tiles (2 x 4).  A stage is 256 k: 256 E4M3 bytes per A row and 128
// E2M1 bytes per B row, 32 KiB each -- the same 64 KiB per stage as the
// W4A4 ring, and the same MFMA time per stage (an instruction with an E4M3
// operand issues at half the E2M1 rate, and the tile has half the outputs).
//   * Operands and scales are fed by direct buffer -> LDS loads
//     (buffer_load_dwordx4 ... lds: lane i's 16 bytes land at the LDS base +
//     16 i), two stage slots ring in LDS, every request covers whole 128-B
//     lines.
//   * A rows (256 B = 16 units of 16 B): unit u of row r sits at
//     u ^ (r & 15); B rows (128 B): unit u at u ^ ((r >> 1) & 7).  Either
//     way the 16 rows that one 16-lane group reads hit distinct banks.
//   * Operands are swapped (B feeds the instruction's first operand), so a
//     lane holds four consecutive output columns.
//   * Scales, tile order, pipelining and the bf16 epilogue (tile staged in
//     LDS, stored in whole 16-byte units) follow the W4A4 ring.
constexpr int kA8M = 128, kA8N = 256;                     // block tile
constexpr int kA8RowA = 256, kA8RowB = 128;               // bytes per row per stage
constexpr int kA8Stage = kA8M * kA8RowA + kA8N * kA8RowB;  // 64 KiB
constexpr int kA8Scale = (kA8M + kA8N) * 16;               // scales of a stage pair

template <int B>
__device__ __forceinline__ uint8_t* a8_codes() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[kA8Stage];
  return buf;
}
template <int B>
__device__ __forceinline__ uint8_t* a8_scales() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[kA8Scale];
  return buf;
}

template <bool kBf16Out>
__global__ __launch_bounds__(512, 1) void k_w4a8_ring(const uint8_t* __restrict__ aq8,
                                                      const uint8_t* __restrict__ as,
                                                      const uint8_t* __restrict__ bq,
                                                      const uint8_t* __restrict__ bs, int64_t m, int64_t n,
                                                      int64_t k, void* __restrict__ c) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it stay scalar
  const int wm = wave >> 2, wn = wave & 3;
  const int half = lane >> 5, r32 = lane & 31;

  // tiles ordered per XCD (contiguous runs of tile ids), four tile rows deep
  const int64_t tm_n = (m + kA8M - 1) / kA8M, tn_n = (n + kA8N - 1) / kA8N;
  const int64_t tiles = tm_n * tn_n;
  int64_t tid_lin = blockIdx.x;
  if (tiles % 8 == 0) tid_lin = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int64_t group = 4;
  const int64_t per_group = group * tn_n;
  const int64_t g0 = (tid_lin / per_group) * group;
  const int64_t gsz = (tm_n - g0) < group ? (tm_n - g0) : group;
  const int64_t tm = g0 + (tid_lin % per_group) % gsz;
  const int64_t tn = (tid_lin % per_group) / gsz;
  const int64_t m0 = tm * kA8M, n0 = tn * kA8N;

  const int64_t kq = k / 2, ks = k / 32;
  const int nstages = (int)(k / 256);  // a multiple of 4
  const int npairs = nstages / 2;
  // rows of this tile that exist (missing rows re-read the last one and are
  // never stored)
  const int rows_a = (int)min((int64_t)kA8M, m - m0), rows_b = (int)min((int64_t)kA8N, n - n0);

  // scale copies, 16 B per row per stage pair, one per wave and no branch
  // (a branch here splits the stage into separate scheduling regions):
  // waves 0-1 copy the 128 A rows, waves 2-5 the 256 B rows, and waves 6-7
  // copy the A rows again (the same bytes to the same place)
  const bool sc_a = wave < 2 || wave >= 6;
  const int srow = sc_a ? 64 * (wave & 1) + lane : 64 * (wave - 2) + lane;
  const int sdst = sc_a ? (64 * (wave & 1)) * 16 : kA8M * 16 + (64 * (wave - 2)) * 16;
  // buffer resources over the tile's row panels (below 2^31 bytes: the
  // launcher takes this kernel for k < 2^24 only)
  const __amdgpu_buffer_rsrc_t rA = panel_rsrc(aq8 + m0 * k, rows_a * k);
  const __amdgpu_buffer_rsrc_t rB = panel_rsrc(bq + n0 * kq, rows_b * kq);
  const __amdgpu_buffer_rsrc_t rS = sc_a ? panel_rsrc(as + m0 * ks, rows_a * ks) : panel_rsrc(bs + n0 * ks, rows_b * ks);
  const unsigned soff_row = (unsigned)(min(srow, sc_a ? rows_a - 1 : rows_b - 1) * ks);
  // code copies: wave w fills A rows 16 w .. 16 w + 15 (4 copies of 4 rows)
  // and B rows 32 w .. 32 w + 31 (4 copies of 8 rows); lane offsets fixed
  // for the k loop, the swizzle applied on the global side
  unsigned offa[4], offb[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int ra = 16 * wave + 4 * j + (lane >> 4);  // ra & 15 == 4 j + lane / 16
    offa[j] = (unsigned)min(ra, rows_a - 1) * (unsigned)k + (unsigned)(((lane & 15) ^ (4 * j + (lane >> 4))) << 4);
    const int rb = 32 * wave + 8 * j + (lane >> 3);  // (rb >> 1) & 7 == (4 j + lane / 16) & 7
    offb[j] = (unsigned)min(rb, rows_b - 1) * (unsigned)kq +
              (unsigned)(((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)) << 4);
  }

  auto issue_codes = [&](auto cb_tag, int s) {
    uint8_t* base = a8_codes<decltype(cb_tag)::value>();
    const unsigned sc = (unsigned)min(s, nstages - 1);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      bdma16(rA, offa[j], sc * kA8RowA, base + (16 * wave + 4 * j) * kA8RowA);
      bdma16(rB, offb[j], sc * kA8RowB, base + kA8M * kA8RowA + (32 * wave + 8 * j) * kA8RowB);
    }
  };
  auto issue_scales = [&](auto sb_tag, int p) {
    uint8_t* sbase = a8_scales<decltype(sb_tag)::value>();
    bdma16(rS, soff_row, (unsigned)min(p, npairs - 1) * 16u, sbase + sdst);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = (f32x16){};

  struct Frag {
    i32x4 a[2][2], b[2];  // a[i][run]: the lane's two 16-k runs of A
  };
  // fragment rows are wm*64 + 32 i + r32 (A) and wn*64 + 32 j + r32 (B):
  // their swizzles depend on r32 only
  const int swa = r32 & 15, swb = (r32 >> 1) & 7;
  const int laneA = (wm * 64 + r32) * kA8RowA, laneB = kA8M * kA8RowA + (wn * 64 + r32) * kA8RowB;
  auto read_frag = [&](auto cb_tag, int kk, Frag& f) {
    const uint8_t* ring = a8_codes<decltype(cb_tag)::value>();
    // A runs: logical units 4 kk + half and 4 kk + 2 + half (physically ^ 2)
    const int ua = ((4 * kk + half) ^ swa) << 4;
    const int ub = ((2 * kk + half) ^ swb) << 4;
#pragma unroll
    for (int j = 0; j < 2; j++) f.b[j] = *(const i32x4*)(ring + laneB + ub + j * 32 * kA8RowB);
#pragma unroll
    for (int i = 0; i < 2; i++) {
      f.a[i][0] = *(const i32x4*)(ring + laneA + i * 32 * kA8RowA + ua);
      f.a[i][1] = *(const i32x4*)(ring + laneA + i * 32 * kA8RowA + (ua ^ 32));
    }
  };
  struct Scales {
    unsigned a[2][2], b[2][2];
  };
  // stage s's scale dwords (dword d = blocks 4d..4d+3 of the stage), pre-
  // shifted for the lane's k half
  auto read_scales = [&](auto sb_tag, int odd, Scales& sc) {
    const unsigned* ss = (const unsigned*)a8_scales<decltype(sb_tag)::value>();
    const int d0 = 2 * odd;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int ra_row = wm * 64 + i * 32 + r32, rb_row = wn * 64 + i * 32 + r32;
#pragma unroll
      for (int d = 0; d < 2; d++) {
        const unsigned va = ss[ra_row * 4 + d0 + d];
        const unsigned vb = ss[kA8M * 4 + rb_row * 4 + d0 + d];
        sc.a[i][d] = half ? (va >> 8) : va;
        sc.b[i][d] = half ? (vb >> 8) : vb;
      }
    }
  };
  auto mma = [&](const Frag& f, const Scales& sc, int kk) {
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const i32x8 fa = {f.a[i][0].x, f.a[i][0].y, f.a[i][0].z, f.a[i][0].w,
                          f.a[i][1].x, f.a[i][1].y, f.a[i][1].z, f.a[i][1].w};
        const i32x8 fb = {f.b[j].x, f.b[j].y, f.b[j].z, f.b[j].w, 0, 0, 0, 0};
        const unsigned sa = sc.a[i][kk >> 1], sb = sc.b[j][kk >> 1];
        if ((kk & 1) == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc[i][j], kFmtFp4, kFmtFp8, 0, sb,
                                                                        0, sa);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc[i][j], kFmtFp4, kFmtFp8, 2, sb,
                                                                        2, sa);
      }
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  Frag f0, f1;
  Scales sc;
  auto stage = [&](auto s_tag, int s) {
    constexpr int S = decltype(s_tag)::value;
    using CB = std::integral_constant<int, S & 1>;
    using NB = std::integral_constant<int, (S + 1) & 1>;
    using NSB = std::integral_constant<int, ((S + 1) >> 1) & 1>;
    // per 64-k step: 6 fragment reads, 4 MFMAs
    read_frag(CB{}, 1, f1);
    mma(f0, sc, 0);
    interleave_reads_mfma<2, 1>();
    read_frag(CB{}, 2, f0);
    mma(f1, sc, 1);
    interleave_reads_mfma<2, 1>();
    read_frag(CB{}, 3, f1);
    mma(f0, sc, 2);
    interleave_reads_mfma<2, 1>();
    // stage s+1 visible before its fragments are read; this stage's slot is
    // refilled with stage s+2 once every wave has finished reading it
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_codes(CB{}, s + 2);
    if constexpr ((S & 1) == 0) issue_scales(std::integral_constant<int, ((S + 2) >> 1) & 1>{}, (s + 2) >> 1);
    __builtin_amdgcn_sched_barrier(0);
    Scales scn;
    read_scales(NSB{}, (S + 1) & 1, scn);
    read_frag(NB{}, 0, f0);
    mma(f1, sc, 3);
    interleave_reads_mfma<4, 1>();
    sc = scn;
  };

  // prologue: stages 0 and 1 and the scales of pair 0 in flight
  issue_codes(C0{}, 0);
  issue_scales(C0{}, 0);
  issue_codes(C1{}, 1);
  wait_vmcnt<8>();  // stage 0 and the scales landed; stage 1 (8 copies) may be in flight
  __builtin_amdgcn_s_barrier();
  read_scales(C0{}, 0, sc);
  read_frag(C0{}, 0, f0);
  for (int s = 0; s < nstages; s += 4) {
    stage(std::integral_constant<int, 0>{}, s);
    stage(std::integral_constant<int, 1>{}, s + 1);
    stage(std::integral_constant<int, 2>{}, s + 2);
    stage(std::integral_constant<int, 3>{}, s + 3);
  }
  wait_vmcnt<0>();  // no copy may still target LDS when the block ends

  if constexpr (kBf16Out) {
    // the 128 x 256 bf16 tile into code slot 0 (512 B per row, 16-byte unit
    // u of row r at u ^ (r & 31)), then stored row by row in whole units
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __syncthreads();
    uint8_t* lo = a8_codes<0>();
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int tr = wm * 64 + i * 32 + r32;
      uint8_t* rowp = lo + tr * 512;
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int tc = wn * 64 + j * 32 + q * 8 + 4 * half;
          const u32x2 o = {f32_to_bf16_rne(acc[i][j][4 * q]) | ((unsigned)f32_to_bf16_rne(acc[i][j][4 * q + 1]) << 16),
                           f32_to_bf16_rne(acc[i][j][4 * q + 2]) | ((unsigned)f32_to_bf16_rne(acc[i][j][4 * q + 3]) << 16)};
          *(u32x2*)(rowp + (((tc >> 3) ^ (tr & 31)) << 4) + 2 * (tc & 7)) = o;
        }
    }
    __syncthreads();
    store_bf16_tile<128, 512>(lo, lo, m0, n0, m, n, (uint16_t*)c);
    return;
  }

#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int64_t row = m0 + wm * 64 + i * 32 + r32;
    if (row >= m) continue;
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int64_t col = n0 + wn * 64 + j * 32 + q * 8 + 4 * half;
        const float vv[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (col + 3 < n) {
          *(f32x4*)((float*)c + row * n + col) = (f32x4){vv[0], vv[1], vv[2], vv[3]};
        } else {
          for (int e = 0; e < 4 && col + e < n; e++) ((float*)c)[row * n + col + e] = vv[e];
        }
      }
  }
}

hipError_t launch_w4a8(const uint8_t* aq8, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                       int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st) {
  if (gemm_skinny_applies(m, k)) return launch_w4a8_skinny(aq8, as, bq, bs, m, n, k, c, bf16_out, st);
  // the ring's per-lane copy offsets are 32-bit: 128 rows * k < 2^32
  if (k % 1024 == 0 && k >= 1024 && k < (1 << 24)) {
    const unsigned tiles = (unsigned)(((m + kA8M - 1) / kA8M) * ((n + kA8N - 1) / kA8N));
    if (bf16_out)
      hipLaunchKernelGGL(k_w4a8_ring<true>, dim3(tiles), dim3(512), 0, st, aq8, as, bq, bs, m, n, k, c);
    else
      hipLaunchKernelGGL(k_w4a8_ring<false>, dim3(tiles), dim3(512), 0, st, aq8, as, bq, bs, m, n, k, c);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 127) / 128));
  if (bf16_out)
    hipLaunchKernelGGL(k_w4a8_direct<true>, grid, dim3(256), 0, st, aq8, as, bq, bs, m, n, k, c);
  else
    hipLaunchKernelGGL(k_w4a8_direct<false>, grid, dim3(256), 0, st, aq8, as, bq, bs, m, n, k, c);
  return hipGetLastError();
}

}  // namespace mxq
