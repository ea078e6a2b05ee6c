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
#include <type_traits>

#include "mxq_device.h"
#include "mxq_gemm_common.h"
#include "mxq_launch.h"

namespace mxq {

// First version: every wave streams its own operand fragments from global
// memory (L2-resident) -- block tile 128 x 128, wave tile 64 x 64 = 2 x 2
// MFMAs per 64-wide k step.
template <int OUT>
__global__ __launch_bounds__(256) void k_w4a4_direct(const uint8_t* __restrict__ aq,
                                                     const uint8_t* __restrict__ as,
                                                     const uint8_t* __restrict__ bq,
                                                     const uint8_t* __restrict__ bs, int64_t m, int64_t n,
                                                     int64_t k, void* __restrict__ c, uint8_t* __restrict__ cs) {
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

  if constexpr (OUT == kOutMx) {
    // bf16 tile staged in LDS, then quantized row-wise (16-byte unit u of
    // tile row r at u ^ (r & 15))
    __shared__ __attribute__((aligned(16))) uint8_t tile[128 * 256];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int tr = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
          const int tc = 64 * wn + 32 * j + r32;
          *(uint16_t*)(tile + tr * 256 + (((tc >> 3) ^ (tr & 15)) << 4) + 2 * (tc & 7)) =
              f32_to_bf16_rne(acc[i][j][r]);
        }
    __syncthreads();
    store_mx_tile<128, 256>(tile, tile, (int64_t)blockIdx.y * 128, (int64_t)blockIdx.x * 128, m, n, (uint8_t*)c, cs);
    return;
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
        if (OUT == kOutBf16)
          ((uint16_t*)c)[rr * n + cc] = f32_to_bf16_rne(acc[i][j][r]);
        else
          ((float*)c)[rr * n + cc] = acc[i][j][r];
      }
    }
}

constexpr int kBM = 256;  // block tile rows of the ring kernel (columns: 256 or 128)
// tile rows per group of the ring kernel's tile order (L2 reuse of B panels)
#ifndef MXQ_W4A4_GROUP
#define MXQ_W4A4_GROUP 4
#endif

// ---------------------------------------------------------------------------
// Ring kernel (k % 1024 == 0).  Block tile 256 x 256; each wave multiplies
// 32 x 32 blocks on v_mfma_scale_f32_32x32x64_f8f6f4 (one lane = 32 k = one
// MX block = one E8M0 operand byte).  Operands are fed by direct
// buffer -> LDS loads (buffer_load_dwordx4 ... lds: lane i's 16 bytes land
// at LDS base + 16 i; the scales by the global-address form), no staging
// registers.  A stage is 256 k = 128 code bytes per row, so every request is
// a whole 128-B line (half-line requests ran at roughly half the L2
// throughput); two stages of 64 KiB ring in LDS.
//   * Operands are swapped (B rows feed the instruction's A side), so a lane
//     holds four consecutive output columns (the fp32 epilogue stores them
//     as one 16-byte write; bf16 and MXFP4 outputs are staged in LDS).
//   * Tiles are ordered per XCD: the blocks an XCD runs take a contiguous
//     run of tile ids, grouped four tile rows deep for L2 reuse.
//   * LDS rows are 128 B; unit u (16 B) of row r sits at u ^ ((r >> 1) & 7),
//     so the 16 rows one 16-lane group reads hit distinct banks.  The
//     swizzle is applied on the global side: lane i of a DMA fills row i / 8,
//     unit i % 8, and fetches logical unit (i % 8) ^ ((row >> 1) & 7).
//   * Fragments are software-pipelined per 64-k step: step kk's MFMAs run
//     while step kk+1's fragments are read; in the last step of a stage the
//     wave waits for the next stage's DMA, meets the other waves at a
//     barrier (without a memory fence, which would drain the prefetch), and
//     only then refills the buffer everyone has finished reading.
//   * E8M0 scales: 16 bytes per row per PAIR of stages, one 16-byte DMA per
//     row (a 4-byte fetch per row and stage made as many L2 requests as all
//     the code bytes), double-buffered by pair.
constexpr int kSB = 128;                   // code bytes per row per stage
// Ring slots: each stage buffer and each scale-pair buffer is its own LDS
// variable, addressed only through compile-time slot indices, so the
// compiler can see that the fragment reads of one slot do not touch the
// slot whose copy is in flight (with one shared array it would wait for
// every outstanding copy before the first read, serializing copy and math).
// A slot holds the A then the B codes of one stage ((256 + BN) rows x 128
// B); a scale slot the A then the B scales of a stage pair (16 B per row).
template <int BN, int B>
__device__ __forceinline__ uint8_t* w4_codes() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[(kBM + BN) * kSB];
  return buf;
}
template <int BN, int B>
__device__ __forceinline__ uint8_t* w4_scales() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[(kBM + BN) * 16];
  return buf;
}

// NWV waves per block: 4 (a 2 x 2 grid of 128 x 128 wave tiles, one wave
// per SIMD) or 8 (2 x 4 of 128 x 64, two waves per SIMD, so one wave's
// MFMAs cover the other's waits).  BN = 128 halves the tile's columns (8
// waves of 128 x 32): twice the tiles where 256 x 256 leaves CUs idle.
#ifndef MXQ_W4A4_WUNI
#define MXQ_W4A4_WUNI 1
#endif
template <int NWV, int OUT, int BN>
__global__ __launch_bounds__(64 * NWV, 1) void k_w4a4_ring(const uint8_t* __restrict__ aq,
                                                           const uint8_t* __restrict__ as,
                                                           const uint8_t* __restrict__ bq,
                                                           const uint8_t* __restrict__ bs, int64_t m, int64_t n,
                                                           int64_t k, void* __restrict__ c,
                                                           uint8_t* __restrict__ cs) {
  static_assert((NWV == 4 && BN == 256) || (NWV == 8 && (BN == 256 || BN == 128)), "tile / waves");
  constexpr int WNC = NWV / 2;        // wave columns
  constexpr int WCOLS = BN / WNC;     // output columns per wave
  constexpr int JB = WCOLS / 32;      // B fragments per wave
  constexpr int RPW = kBM / NWV;      // A rows each wave copies
  constexpr int CJ = RPW / 8;         // A copy instructions per wave
  constexpr int RPWB = BN / NWV;      // B rows each wave copies
  constexpr int CJB = RPWB / 8;       // B copy instructions per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = MXQ_W4A4_WUNI ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;  // uniform
  const int wm = wave / WNC, wn = wave % WNC;
  const int half = lane >> 5, r32 = lane & 31;

  const int64_t tm_n = (m + kBM - 1) / kBM, tn_n = (n + BN - 1) / BN;
  const int64_t tiles = tm_n * tn_n;
  int64_t tid_lin = blockIdx.x;
  if (tiles % 8 == 0) tid_lin = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int64_t group = MXQ_W4A4_GROUP;
  const int64_t per_group = group * tn_n;
  const int64_t g0 = (tid_lin / per_group) * group;
  const int64_t gsz = (tm_n - g0) < group ? (tm_n - g0) : group;
  const int64_t tm = g0 + (tid_lin % per_group) % gsz;
  const int64_t tn = (tid_lin % per_group) / gsz;
  const int64_t m0 = tm * kBM, n0 = tn * BN;

  const int64_t kq = k / 2, ks = k / 32;
  const int nstages = (int)(k / 256);  // a multiple of 4 (k % 1024 == 0)
  const int npairs = nstages / 2;

  // rows of this tile that exist (the last tile may be partial: its missing
  // rows re-read the last row and are never stored)
  const int rows_a = (int)min((int64_t)kBM, m - m0), rows_b = (int)min((int64_t)BN, n - n0);
  // scale copies: 16 B per row per stage pair; with 4 waves each wave copies
  // 64 rows of A and of B, with 8 waves waves 0-3 copy A and 4-7 copy B
  // (with BN = 128, waves 6-7 repeat waves 4-5: the same bytes to the same
  // place, so every wave issues one copy)
  const int srow = NWV == 4 ? 64 * wave + lane : 64 * ((wave & 3) % (wave < 4 ? 4 : BN / 64)) + lane;
  // codes through buffer resources over the tile's row panels (the launcher
  // keeps every panel below 2^31 bytes); per-lane offsets fixed for the k loop
  const __amdgpu_buffer_rsrc_t rA = panel_rsrc(aq + m0 * kq, rows_a * kq);
  const __amdgpu_buffer_rsrc_t rB = panel_rsrc(bq + n0 * kq, rows_b * kq);
  const uint8_t* gsa = as + min(m0 + srow, m - 1) * ks;
  const uint8_t* gsb = bs + min(n0 + srow, n - 1) * ks;
  // lane offsets of the CJ code copies per operand (fixed for the k loop)
  unsigned offa[CJ], offb[CJB];
#pragma unroll
  for (int j = 0; j < CJ; j++) {
    // lane -> LDS row RPW w + 8j + lane/8, physical unit lane%8, logical unit
    // (lane%8) ^ ((row >> 1) & 7) = (lane%8) ^ ((4j + lane/16) & 7)
    const int row = RPW * wave + 8 * j + (lane >> 3);
    const unsigned cu16 = (unsigned)(((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)) << 4);
    offa[j] = (unsigned)min(row, rows_a - 1) * (unsigned)kq + cu16;
  }
#pragma unroll
  for (int j = 0; j < CJB; j++) {
    // B rows RPWB w + 8j + lane/8; RPWB w is a multiple of 16, so the swizzle
    // unit is the same expression as for A
    const int row = RPWB * wave + 8 * j + (lane >> 3);
    const unsigned cu16 = (unsigned)(((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)) << 4);
    offb[j] = (unsigned)min(row, rows_b - 1) * (unsigned)kq + cu16;
  }

  // codes of stage s into code slot CB: 2 CJ copies per wave (a stage past
  // the end is clamped to the last one: a re-read into a slot nobody reads)
  auto issue_codes = [&](auto cb_tag, int s) {
    uint8_t* base = w4_codes<BN, decltype(cb_tag)::value>();
    const unsigned soff = (unsigned)min(s, nstages - 1) * kSB;
#pragma unroll
    for (int j = 0; j < CJ; j++) bdma16(rA, offa[j], soff, base + (RPW * wave + 8 * j) * kSB);
#pragma unroll
    for (int j = 0; j < CJB; j++) bdma16(rB, offb[j], soff, base + kBM * kSB + (RPWB * wave + 8 * j) * kSB);
  };
  // scales of stage pair p into scale slot SB: 16 B per row (2 copies per
  // wave with 4 waves, 1 with 8)
  auto issue_scales = [&](auto sb_tag, int p) {
    uint8_t* sbase = w4_scales<BN, decltype(sb_tag)::value>();
    const int pc = min(p, npairs - 1);
    if (NWV == 4) {
      dma16(gsa + (int64_t)pc * 16, sbase + (64 * wave) * 16);
      dma16(gsb + (int64_t)pc * 16, sbase + kBM * 16 + (64 * wave) * 16);
    } else if (wave < 4) {
      dma16(gsa + (int64_t)pc * 16, sbase + (64 * wave) * 16);
    } else {
      dma16(gsb + (int64_t)pc * 16, sbase + kBM * 16 + (64 * ((wave - 4) % (BN / 64))) * 16);
    }
  };

  f32x16 acc[4][JB];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < JB; j++) acc[i][j] = (f32x16){};

  struct Frag {
    i32x4 a[4], b[JB];
  };
  // fragments of 64-k step kk (0..3) of the stage in code slot CB.
  // Fragment addresses factor: row = w*128 + i*32 + r32 has (row >> 1) & 7
  // == (r32 >> 1) & 7 for every i and for A and B alike, so one physical
  // unit per k step serves all eight fragments and i is an immediate offset.
  const int swz = (r32 >> 1) & 7;
  const int laneA = (wm * 128 + r32) * kSB, laneB = kBM * kSB + (wn * WCOLS + r32) * kSB;
  auto read_frag = [&](auto cb_tag, int kk, Frag& f) {
    const uint8_t* ring = w4_codes<BN, decltype(cb_tag)::value>();
    const int unit16 = ((kk * 2 + half) ^ swz) << 4;
    const uint8_t* pa = ring + laneA + unit16;
    const uint8_t* pb = ring + laneB + unit16;
    // B fragments first: the first MFMAs of a step need every B fragment
    // but only the first A fragment (the MFMA order is A-outer, B-inner)
#pragma unroll
    for (int j = 0; j < JB; j++) f.b[j] = *(const i32x4*)(pb + j * 32 * kSB);
#pragma unroll
    for (int i = 0; i < 4; i++) f.a[i] = *(const i32x4*)(pa + i * 32 * kSB);
  };
  // scale dwords of this lane's rows (dword d = blocks 4d..4d+3 of the stage),
  // pre-shifted for the lane's k half
  struct Scales {
    unsigned a[4][2], b[JB][2];
  };
  // stage s's scale dwords: dwords 2(s&1), 2(s&1)+1 of the pair in slot SB
  auto read_scales = [&](auto sb_tag, int odd, Scales& sc) {
    const unsigned* ss = (const unsigned*)w4_scales<BN, decltype(sb_tag)::value>();
    const int d0 = 2 * odd;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int ra_row = wm * 128 + i * 32 + r32;
      const int rb_row = wn * WCOLS + i * 32 + r32;
#pragma unroll
      for (int d = 0; d < 2; d++) {
        const unsigned va = ss[ra_row * 4 + d0 + d];
        sc.a[i][d] = half ? (va >> 8) : va;
        if (i < JB) {
          const unsigned vb = ss[kBM * 4 + rb_row * 4 + d0 + d];
          sc.b[i][d] = half ? (vb >> 8) : vb;
        }
      }
    }
  };
  auto mma = [&](const Frag& f, const Scales& sc, int kk) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < JB; j++) {
        const i32x8 fa = {f.a[i].x, f.a[i].y, f.a[i].z, f.a[i].w, 0, 0, 0, 0};
        const i32x8 fb = {f.b[j].x, f.b[j].y, f.b[j].z, f.b[j].w, 0, 0, 0, 0};
        const unsigned sa = sc.a[i][kk >> 1], sb = sc.b[j][kk >> 1];
        if ((kk & 1) == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc[i][j], 4, 4, 0, sb, 0, sa);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc[i][j], 4, 4, 2, sb, 2, sa);
      }
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  Frag f0, f1;
  Scales sc;
  // one stage s (S = s % 4): code slot S & 1, scale slot S >> 1.  Straight-
  // line code: the copies, the waits and the reads of the next stage have
  // no branch between them.
  auto stage = [&](auto s_tag, int s) {
    constexpr int S = decltype(s_tag)::value;
    using CB = std::integral_constant<int, S & 1>;
    using NB = std::integral_constant<int, (S + 1) & 1>;
    using NSB = std::integral_constant<int, ((S + 1) >> 1) & 1>;
    // reads per k step: 4 + JB fragments; MFMAs: 4 JB
    constexpr int RG = (4 + JB + 3) / 4, MG = JB;
    read_frag(CB{}, 1, f1);
    mma(f0, sc, 0);
    interleave_reads_mfma<RG, MG>();
    read_frag(CB{}, 2, f0);
    mma(f1, sc, 1);
    interleave_reads_mfma<RG, MG>();
    read_frag(CB{}, 3, f1);
    mma(f0, sc, 2);
    interleave_reads_mfma<RG, MG>();
    // stage s+1 must be visible before its fragments are read, and this
    // stage's slot is refilled with stage s+2 once every wave has finished
    // reading it (this wave's reads: lgkmcnt(0); everyone's: the barrier)
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    // the copies go out right after the barrier (the scheduler would sink
    // them to the end of the stage, shrinking the time they have to land)
    __builtin_amdgcn_sched_barrier(0);
    issue_codes(CB{}, s + 2);
    if constexpr ((S & 1) == 0) issue_scales(std::integral_constant<int, ((S + 2) >> 1) & 1>{}, (s + 2) >> 1);
    __builtin_amdgcn_sched_barrier(0);
    Scales scn;
    read_scales(NSB{}, (S + 1) & 1, scn);
    read_frag(NB{}, 0, f0);
    mma(f1, sc, 3);
    interleave_reads_mfma<RG + 1, MG>();
    sc = scn;
  };

  // prologue: stages 0 and 1 and the scales of pair 0 in flight
  issue_codes(C0{}, 0);
  issue_scales(C0{}, 0);
  issue_codes(C1{}, 1);
  wait_vmcnt<CJ + CJB>();  // stage 0 and the scales landed; stage 1 (CJ + CJB copies) may be in flight
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

  if constexpr (OUT == kOutMx || OUT == kOutBf16) {
    // the bf16 tile into the two code slots (idle now that every wave has
    // read its last fragments): rows 0..127 in slot 0, 128..255 in slot 1,
    // 2 BN bytes per row, 16-byte unit u of row r at u ^ (r % (BN / 8)); then
    // stored row by row in whole 16-byte units (bf16 output, a lane's own
    // 8-byte pieces wrote partial lines) or quantized (MXFP4 output)
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __syncthreads();
    constexpr int TROW = 2 * BN, TU = BN / 8;  // tile row bytes, 16-byte units per row
    uint8_t* lo = w4_codes<BN, 0>();
    uint8_t* hi = w4_codes<BN, 1>();
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int tr = wm * 128 + i * 32 + r32;
      uint8_t* rowp = (tr < 128 ? lo : hi) + (tr & 127) * TROW;
#pragma unroll
      for (int j = 0; j < JB; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int tc = wn * WCOLS + j * 32 + q * 8 + 4 * half;
          const u32x2 o = {f32_to_bf16_rne(acc[i][j][4 * q]) | ((unsigned)f32_to_bf16_rne(acc[i][j][4 * q + 1]) << 16),
                           f32_to_bf16_rne(acc[i][j][4 * q + 2]) | ((unsigned)f32_to_bf16_rne(acc[i][j][4 * q + 3]) << 16)};
          *(u32x2*)(rowp + (((tc >> 3) ^ (tr % TU)) << 4) + 2 * (tc & 7)) = o;
        }
    }
    __syncthreads();
    if constexpr (OUT == kOutMx)
      store_mx_tile<256, TROW>(lo, hi, m0, n0, m, n, (uint8_t*)c, cs);
    else
      store_bf16_tile<256, TROW>(lo, hi, m0, n0, m, n, (uint16_t*)c);
    return;
  }

#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t row = m0 + wm * 128 + i * 32 + r32;
    if (row >= m) continue;
#pragma unroll
    for (int j = 0; j < JB; j++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int64_t col = n0 + wn * WCOLS + j * 32 + q * 8 + 4 * half;
        const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                    v3 = acc[i][j][4 * q + 3];
        if (col + 3 < n) {
          if (OUT == kOutBf16) {
            u32x2 o = {f32_to_bf16_rne(v0) | ((unsigned)f32_to_bf16_rne(v1) << 16),
                       f32_to_bf16_rne(v2) | ((unsigned)f32_to_bf16_rne(v3) << 16)};
            *(u32x2*)((uint16_t*)c + row * n + col) = o;
          } else {
            *(f32x4*)((float*)c + row * n + col) = (f32x4){v0, v1, v2, v3};
          }
        } else {
          const float vv[4] = {v0, v1, v2, v3};
          for (int e = 0; e < 4 && col + e < n; e++) {
            if (OUT == kOutBf16)
              ((uint16_t*)c)[row * n + col + e] = f32_to_bf16_rne(vv[e]);
            else
              ((float*)c)[row * n + col + e] = vv[e];
          }
        }
      }
    }
  }
}

#ifndef MXQ_W4A4_RING_WAVES
#define MXQ_W4A4_RING_WAVES 8
#endif
constexpr int kRingWaves = MXQ_W4A4_RING_WAVES;
// 256 x 128 tiles when 256 x 256 ones would fill at most half the CUs.
// Measured on a 28672 x 8192 weight: m = 160-256 (112 wide tiles) 65-72 ->
// 50-55 us; m = 384-512 (224 wide tiles) 68-76 us wide but 90-100 us narrow
// (the narrow tile copies each A panel twice as often and reads more LDS per
// MFMA).
#ifndef MXQ_W4A4_NARROW_BELOW
#define MXQ_W4A4_NARROW_BELOW 129
#endif

// Returns the launch status (the skinny launcher reads, and so clears, the
// error state itself; its status is passed on as is).
template <int OUT>
static hipError_t launch_w4a4_out(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                                  int64_t m, int64_t n, int64_t k, void* c, uint8_t* cs, hipStream_t st) {
  if (OUT != kOutMx && gemm_skinny_applies(m, k))
    return launch_w4a4_skinny(aq, as, bq, bs, m, n, k, c, OUT == kOutBf16, st);
  // the ring addresses its row panels with 32-bit offsets: 256 rows * k/2
  // bytes stay below 2^31 for k < 2^24
  if (k % 1024 == 0 && k >= 1024 && k < (1 << 24)) {
    const int64_t tm_n = (m + kBM - 1) / kBM;
    // 256-column tiles unless they would leave most CUs idle: then
    // 128-column tiles, twice as many
    if constexpr (kRingWaves == 8) {
      if (tm_n * ((n + 255) / 256) < MXQ_W4A4_NARROW_BELOW) {
        const unsigned tiles = (unsigned)(tm_n * ((n + 127) / 128));
        hipLaunchKernelGGL((k_w4a4_ring<8, OUT, 128>), dim3(tiles), dim3(512), 0, st, aq, as, bq, bs, m, n, k, c, cs);
        return hipGetLastError();
      }
    }
    const unsigned tiles = (unsigned)(tm_n * ((n + 255) / 256));
    hipLaunchKernelGGL((k_w4a4_ring<kRingWaves, OUT, 256>), dim3(tiles), dim3(64 * kRingWaves), 0, st, aq, as, bq,
                       bs, m, n, k, c, cs);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 127) / 128));
  hipLaunchKernelGGL(k_w4a4_direct<OUT>, grid, dim3(256), 0, st, aq, as, bq, bs, m, n, k, c, cs);
  return hipGetLastError();
}

hipError_t launch_w4a4(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                       int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st) {
  return bf16_out ? launch_w4a4_out<kOutBf16>(aq, as, bq, bs, m, n, k, c, nullptr, st)
                  : launch_w4a4_out<kOutF32>(aq, as, bq, bs, m, n, k, c, nullptr, st);
}

hipError_t launch_w4a4_mx(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                          int64_t n, int64_t k, uint8_t* cq, uint8_t* cs, hipStream_t st) {
  return launch_w4a4_out<kOutMx>(aq, as, bq, bs, m, n, k, cq, cs, st);
}

}  // namespace mxq
