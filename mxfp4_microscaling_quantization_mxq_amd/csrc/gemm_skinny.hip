// gemm_skinny.hip -- block-scaled MFMA products with few activation rows
// (m <= 128), MXFP4 weights times MXFP4 (W4A4) or MXFP8 (W4A8)
// activations.  The weight stream decides the time, so the kernel is laid
// out like the W4A16 decode ring rather than like an output tile.
//
// A 256 x 256 output tile spends the same MFMA schedule on 16 activation
// rows as on 256, and a 28672-row weight gives it only 112 tiles for 256
// CUs; measured, the W4A4 and W4A8 tile kernels took 53-69 us at every
// m <= 256 on a 28672 x 8192 MXFP4 weight, against about 21 us for the
// weight read itself.  Batch size picks the kernel ["FP4 quantization
// analysis" page, sec. 5.2: small batches and large ones use different GEMM
// back ends].
//
// Instruction: V_MFMA_SCALE_F32_16X16X128_F8F6F4 with the activations as
// operand A (E2M1 or E4M3) and the weights as operand B (E2M1).  Lane l
// holds row l % 16 of its operand in lane group g = l / 16:
//   * E2M1: one 32-element block of the 128-k step (16 bytes, element 2j in
//     the low nibble of byte j, as stored);
//   * E4M3: k = 16 g .. 16 g + 15 (bytes 0-15) and 64 + 16 g .. +15 (bytes
//     16-31) of the step, which is the E4M3 operand of the 32x32x64 form
//     (measured) spread over four lane groups;
// plus the E8M0 byte of block g of the step on either side.  The 16 x 16
// fp32 result sits in lane l at column l % 16, rows 4 g + r of register r.
// Step i of a stage covers stage k 128 i .. 128 i + 127 in order, so the
// instruction's groups of 8 consecutive k are 8 consecutive k of the
// operands (the E4M3 x E2M1 group sums are truncated; see the W4A8 entry
// point).
//
//   * Block = NW waves; wave w owns weight rows n0 + 16 w .. +16 for all of
//     k, which runs in stages of KS = 512 or 256 through an NR-deep LDS ring
//     filled by buffer -> LDS copies.
//   * The activation rows' codes and scales of a stage (MT rows, shared by
//     all waves) ride in the same ring slot.  Every wave issues the same
//     number of copies; surplus ones land in scratch rows, so the wait
//     counts are compile-time constants.
//   * Activation rows m..MT-1 of the operand hold stale or clamped data;
//     they only reach output rows that are never stored.
//   * LDS swizzle (applied on the global side): 16-byte unit v of row r at
//     slot v ^ (r % S), S = min(16, units per row).  Any 8 consecutive lanes
//     of a fragment read hit 8 distinct bank groups.
//   * One s_barrier per stage, after the wave's own copies have landed.
//   * Blocks start their k loop at staggered k (skinny_rotation).
#include <type_traits>

#include "mxq_device.h"
#include "mxq_gemm_common.h"
#include "mxq_launch.h"

namespace mxq {

// Stage geometry for KS k per stage (512 or 256) and activation format.
template <int KS, bool kFp8>
struct SkGeom {
  static constexpr int RowB = KS / 2;               // E2M1 weight code bytes per row
  static constexpr int U = RowB / 16;               // weight units per row (16 or 8)
  static constexpr int RPI = 64 / U;                // weight rows per 1-KiB copy
  static constexpr int XRowB = kFp8 ? KS : KS / 2;  // activation code bytes per row
  static constexpr int XU = XRowB / 16;             // activation units per row
  static constexpr int XRPI = 64 / XU;              // activation rows per 1-KiB copy
  static constexpr int ScB = KS / 32;               // scale bytes per row
  static constexpr int LPR = ScB / 4;               // lanes per row of a scale copy (4-byte lanes)
  static constexpr int STEPS = KS / 128;            // MFMA steps per stage
};
constexpr int swz(int units) { return units < 16 ? units : 16; }

// First stage of a block's k loop: blocks start at staggered k, (block / 8)
// mod (k / 512) chunks of 512, so that the blocks resident at one time read
// different column ranges.  Counted in 512-k chunks, the k order of every
// output is the same for either stage length.
template <int KS>
__device__ __forceinline__ int skinny_rotation(int64_t k) {
  return (int)((blockIdx.x / 8) % (unsigned)(k / 512)) * (512 / KS);
}

// One ring slot.  Each slot is its own LDS variable and every slot index is
// a compile-time constant, so the compiler can tell that reads of one slot
// do not touch the slots whose copies are in flight.
template <int MT, int NW, int KS, bool kFp8, bool RS>
struct SkSlot {
  using G = SkGeom<KS, kFp8>;
  uint8_t w[16 * NW * G::RowB];          // weight codes
  uint8_t x[(MT + G::XRPI) * G::XRowB];  // activation codes, one copy's worth of scratch rows
  // Scales: a 256-byte region per 16 rows (one 64-lane dword copy), row r
  // of a group at (r % 16) * ScB; with 8 scale bytes per row the upper half
  // of a region is scratch.  (Resident scale rows: unused.)
  uint8_t ws[RS ? 16 : NW * 256];                // weight scales
  uint8_t xs[RS ? 16 : (MT / 16 + 1) * 256];     // activation scales, one scratch region
};
template <int MT, int NW, int KS, bool kFp8, bool RS, int B>
__device__ __forceinline__ SkSlot<MT, NW, KS, kFp8, RS>& sk_slot() {
  __shared__ __attribute__((aligned(1024))) SkSlot<MT, NW, KS, kFp8, RS> slot;
  return slot;
}
// Longest k whose scale rows the ring keeps resident in LDS.
constexpr int kSkResK = 8192;

#ifndef MXQ_SK_WUNI
#define MXQ_SK_WUNI 1
#endif
template <bool kFp8, int MT, int NW, int NR, int KS, bool RS, bool kBf16Out>
__global__ __launch_bounds__(64 * NW, 1) void k_gemm_skinny(const uint8_t* __restrict__ aq,
                                                           const uint8_t* __restrict__ as,
                                                           const uint8_t* __restrict__ bq,
                                                           const uint8_t* __restrict__ bs, int64_t m,
                                                           int64_t n, int64_t k, void* __restrict__ c) {
  using G = SkGeom<KS, kFp8>;
  using Slot = SkSlot<MT, NW, KS, kFp8, RS>;
  constexpr int RB = 16 * NW;                        // weight rows per block
  constexpr int MTT = MT / 16;                       // 16-row activation tiles
  constexpr int WC = 16 / G::RPI;                    // weight code copies per wave
  constexpr int XC = (MT / G::XRPI + NW - 1) / NW;   // activation code copies per wave
  constexpr int XS = (MT / 16 + NW - 1) / NW;        // activation scale copies per wave (16 rows each)
  constexpr int D = WC + (RS ? 0 : 1 + XS) + XC;     // copies per wave per stage
  constexpr int WSW = swz(G::U), XSW = swz(G::XU);   // swizzle periods
  static_assert(MT % 16 == 0 && NR >= 2 && NR <= 4 && (NR - 2) * D < 64, "tile / ring depth / vmcnt range");
  // the wave index in a scalar register: the branches on it stay scalar
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = MXQ_SK_WUNI ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  // activation copy a goes to wave a mod NW: up to 16 rows, a wave whose
  // last slot has no real rows skips it and waits on one copy fewer (see the
  // decode ring); taller tiles keep padding with a re-read (the branch costs
  // them registers, 48 B of spill at 128 rows)
  const bool xfull = MT > 16 || wave + NW * (XC - 1) < MT / G::XRPI;
  const int64_t n0 = (int64_t)blockIdx.x * RB;
  const int rows_w = (int)min((int64_t)RB, n - n0);
  const int64_t kq = k / 2, ks = k / 32, kx = kFp8 ? k : k / 2;
  const int nst = (int)(k / KS);
  const int rot = skinny_rotation<KS>(k);
  // absolute stage of loop stage s (a stage past the end is clamped to the last)
  auto stage_of = [&](int s) -> unsigned {
    const int sl0 = min(s, nst - 1);
    return (unsigned)(sl0 + rot < nst ? sl0 + rot : sl0 + rot - nst);
  };
  // Resident scale rows (k <= kSkResK, at most 16 activation rows): each
  // wave's 16 weight rows x ks E8M0 bytes and the block's MT activation rows
  // x ks sit in LDS for the whole k loop, rows padded by 16 B (a fragment
  // read's 16 rows fall in distinct bank groups), instead of two small
  // per-stage scale copies.
  static_assert(!RS || MT <= 16, "resident activation scales: one 16-row tile");
  constexpr int KSMAX = kSkResK / 32;                // scale bytes per row, at most
  constexpr int PU = KSMAX / 64;                     // 16-byte units per lane (weight rows), at most
  __shared__ __attribute__((aligned(16))) uint8_t wres[RS ? NW * 16 * (KSMAX + 16) : 16];
  __shared__ __attribute__((aligned(16))) uint8_t xres[RS ? MT * (KSMAX + 16) : 16];
  const int rsp = (int)ks + 16;                      // LDS pitch of a scale row
  const int upr = (int)(ks >> 4);                    // 16-byte units per scale row

  // Lane offsets of the copies, fixed for the whole k loop (a stage only
  // moves the uniform offset).  Rows past the operand are clamped to its
  // last row: the copy stays in bounds and fills an LDS row nobody stores.
  unsigned offw[WC], offx[XC], offxs[XS];
  int dx[XC], dxs[XS];
#pragma unroll
  for (int q = 0; q < WC; q++) {
    const int row = 16 * wave + G::RPI * q + lane / G::U;
    const unsigned unit = (unsigned)((lane % G::U) ^ (row % WSW));
    offw[q] = (unsigned)min(row, rows_w - 1) * (unsigned)kq + (unit << 4);
  }
  // scale copies: 4 bytes per lane; lane i takes row (i mod 16 LPR) / LPR of
  // the group, dword i mod LPR, so lanes past 16 LPR repeat the group into
  // the region's scratch half
  const int srow = (lane % (16 * G::LPR)) / G::LPR;
  const unsigned spart = 4u * (unsigned)(lane % G::LPR);
  const unsigned offws = (unsigned)min(16 * wave + srow, rows_w - 1) * (unsigned)ks + spart;
#pragma unroll
  for (int j = 0; j < XC; j++) {
    const int a = wave + NW * j;  // copy slot (wave-uniform): activation rows XRPI a ..
    const int row = G::XRPI * a + lane / G::XU;
    const unsigned unit = (unsigned)((lane % G::XU) ^ (row % XSW));
    offx[j] = (unsigned)min((int64_t)row, m - 1) * (unsigned)kx + (unit << 4);
    dx[j] = (G::XRPI * a < MT ? G::XRPI * a : MT) * G::XRowB;
  }
#pragma unroll
  for (int j = 0; j < XS; j++) {
    const int a = wave + NW * j;  // activation rows 16a .. 16a+15
    const int row = 16 * a + srow;
    offxs[j] = (unsigned)min((int64_t)row, m - 1) * (unsigned)ks + spart;
    dxs[j] = (16 * a < MT ? a : MT / 16) * 256;
  }
  const __amdgpu_buffer_rsrc_t rw = panel_rsrc(bq + n0 * kq, rows_w * kq);
  const __amdgpu_buffer_rsrc_t rws = panel_rsrc(bs + n0 * ks, rows_w * ks);
  const __amdgpu_buffer_rsrc_t rx = panel_rsrc(aq, m * kx);
  const __amdgpu_buffer_rsrc_t rxs = panel_rsrc(as, m * ks);

  // Copies of stage s into ring slot B.  A stage past the end is clamped to
  // the last one (a re-read into a slot nobody reads), so every step issues
  // the same copies.
  auto issue = [&](auto slot_tag, int s) {
    constexpr int B = decltype(slot_tag)::value;
    Slot& sl = sk_slot<MT, NW, KS, kFp8, RS, B>();
    const unsigned sc = stage_of(s);
#pragma unroll
    for (int q = 0; q < WC; q++)
      bdma16_nt(rw, offw[q], sc * G::RowB, sl.w + (16 * wave + G::RPI * q) * G::RowB);
    if constexpr (!RS) bdma4(rws, offws, sc * G::ScB, sl.ws + 256 * wave);
#pragma unroll
    for (int j = 0; j < XC; j++)
      if (j < XC - 1 || xfull) bdma16(rx, offx[j], sc * G::XRowB, sl.x + dx[j]);
    if constexpr (!RS) {
#pragma unroll
      for (int j = 0; j < XS; j++) bdma4(rxs, offxs[j], sc * G::ScB, sl.xs + dxs[j]);
    }
  };

  f32x4 acc[MTT];
#pragma unroll
  for (int t = 0; t < MTT; t++) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int wrow = 16 * wave + col;  // this lane's block weight row
  // scale bytes of a row as words: word i holds blocks 4i .. 4i+3
  auto scale_words = [&](const uint8_t* p, unsigned (&wds)[G::STEPS]) {
    if constexpr (G::STEPS == 4) {
      const u32x4 v = *(const u32x4*)p;
      wds[0] = v.x; wds[1] = v.y; wds[2] = v.z; wds[3] = v.w;
    } else {
      const u32x2 v = *(const u32x2*)p;
      wds[0] = v.x; wds[1] = v.y;
    }
  };
  // activation fragment of step i from an activation row r, r % 16 == col
  auto x_fragment = [&](const uint8_t* row, int i) -> i32x8 {
    if constexpr (kFp8) {
      const u32x4 lo = *(const u32x4*)(row + (((8 * i + g) ^ (col % XSW)) << 4));
      const u32x4 hi = *(const u32x4*)(row + (((8 * i + 4 + g) ^ (col % XSW)) << 4));
      return (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      const u32x4 v = *(const u32x4*)(row + (((4 * i + g) ^ (col % XSW)) << 4));
      return (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
  };
  auto compute = [&](auto slot_tag, unsigned sc) {
    constexpr int B = decltype(slot_tag)::value;
    const Slot& sl = sk_slot<MT, NW, KS, kFp8, RS, B>();
    unsigned wss[G::STEPS], xss[MTT][G::STEPS];
    if constexpr (RS) {
      scale_words(wres + wrow * rsp + sc * G::ScB, wss);
#pragma unroll
      for (int t = 0; t < MTT; t++) scale_words(xres + (16 * t + col) * rsp + sc * G::ScB, xss[t]);
    } else {
      scale_words(sl.ws + 256 * wave + col * G::ScB, wss);
#pragma unroll
      for (int t = 0; t < MTT; t++) scale_words(sl.xs + 256 * t + col * G::ScB, xss[t]);
    }
#pragma unroll
    for (int i = 0; i < G::STEPS; i++) {
      const int wslot = ((4 * i + g) ^ (col % WSW)) << 4;  // weight unit 4i+g of a row r, r % 16 == col
      const u32x4 cw = *(const u32x4*)(sl.w + wrow * G::RowB + wslot);
      const i32x8 wf = {(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
      const int sw = (int)((wss[i] >> (8 * g)) & 0xFFu);
#pragma unroll
      for (int t = 0; t < MTT; t++) {
        const i32x8 xf = x_fragment(sl.x + (16 * t + col) * G::XRowB, i);
        const int sx = (int)((xss[t][i] >> (8 * g)) & 0xFFu);
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xf, wf, acc[t], kFp8 ? kFmtFp8 : kFmtFp4, kFmtFp4,
                                                                  0, sx, 0, sw);
      }
    }
  };

  // One stage: wait for its copies (NR - 2 later stages may stay in
  // flight) and for this wave's reads of the slot about to be refilled,
  // meet the other waves, refill, multiply.
  auto step = [&](auto slot_tag, int s) {
    constexpr int B = decltype(slot_tag)::value;
    constexpr int N = (NR - 2) * D, N1 = (NR - 2) * (D - 1);
    if (xfull)
      __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    else
      __builtin_amdgcn_s_waitcnt((N1 & 15) | ((N1 >> 4) << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    issue(std::integral_constant<int, (B + NR - 1) % NR>{}, s + NR - 1);
    if (s < nst) compute(slot_tag, stage_of(s));
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1 % NR>;
  using I2 = std::integral_constant<int, 2 % NR>;
  using I3 = std::integral_constant<int, 3 % NR>;
  // resident scales: PU loads per lane of the wave's weight scale rows
  // (units past its 16 rows re-read a valid unit and are dropped) and one
  // load per thread of the activation scale rows, before the ring's copies
  u32x4 wsv[RS ? PU : 1], xsv = {0u, 0u, 0u, 0u};
  if constexpr (RS) {
#pragma unroll
    for (int p = 0; p < PU; p++) {
      const int i = lane + 64 * p;
      const int r = i / upr, cu = i - r * upr;
      const int row = min(16 * wave + min(r, 15), rows_w - 1);
      wsv[p] = *(const u32x4*)(bs + (n0 + row) * ks + 16 * cu);
    }
    const int r = min(tid / upr, MT - 1), cu = tid - (tid / upr) * upr;
    xsv = *(const u32x4*)(as + min((int64_t)r, m - 1) * ks + 16 * cu);
  }
  issue(I0{}, 0);
  if (NR > 2) issue(I1{}, 1);
  if (NR > 3) issue(I2{}, 2);
  if constexpr (RS) {
    // the scale loads are older than the NR - 1 stages of copies in flight;
    // the first stage's barrier publishes the activation scales
    if (xfull)
      wait_vmcnt<(NR - 1) * D>();
    else
      wait_vmcnt<(NR - 1) * (D - 1)>();
#pragma unroll
    for (int p = 0; p < PU; p++) {
      const int i = lane + 64 * p;
      const int r = i / upr, cu = i - r * upr;
      if (r < 16) *(u32x4*)(wres + (16 * wave + r) * rsp + 16 * cu) = wsv[p];
    }
    if (tid < MT * upr) *(u32x4*)(xres + (tid / upr) * rsp + 16 * (tid - (tid / upr) * upr)) = xsv;
  }
  step(I0{}, 0);
  for (int s = 1; s < nst; s += NR) {
    step(I1{}, s);
    if (NR > 2) step(I2{}, s + 1);
    if (NR > 3) step(I3{}, s + 2);
    step(I0{}, s + NR - 1);
  }
  wait_vmcnt<0>();

  // lane holds c[16t + 4g + e][n0 + wrow]
  const int64_t nn = n0 + wrow;
  if (nn < n) {
#pragma unroll
    for (int t = 0; t < MTT; t++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int64_t mm = 16 * t + 4 * g + e;
        if (mm >= m) continue;
        if (kBf16Out)
          ((uint16_t*)c)[mm * n + nn] = f32_to_bf16_rne(acc[t][e]);
        else
          ((float*)c)[mm * n + nn] = acc[t][e];
      }
  }
}

template <bool kFp8, int MT, int NW, int NR, int KS, bool RS = false>
static void launch_sk(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                      int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st) {
  const dim3 grid((unsigned)((n + 16 * NW - 1) / (16 * NW)));
  if (bf16_out)
    hipLaunchKernelGGL((k_gemm_skinny<kFp8, MT, NW, NR, KS, RS, true>), grid, dim3(64 * NW), 0, st, aq, as, bq, bs,
                       m, n, k, c);
  else
    hipLaunchKernelGGL((k_gemm_skinny<kFp8, MT, NW, NR, KS, RS, false>), grid, dim3(64 * NW), 0, st, aq, as, bq, bs,
                       m, n, k, c);
}

// ---------------------------------------------------------------------------
// W4A4 / W4A8 with the activations quantized in the kernel (MXFP4 or MXFP8
// of bf16 x, with the quantizers of mxq_quantize / mxq_quantize_fp8): the
// bf16 activation rows of a stage ride in the ring instead of codes, and
// the block quantizes them once per stage into a single tile that the MFMAs
// then read exactly as above.
//   * After the stage barrier and the refill copies, lane q of the block
//     takes MX blocks q, q + 64 NW, ... of the stage (one whole 32-element
//     block per lane: mx_quantize_lane_bf16 / mx8_quantize_lane_bf16),
//     writes its 16 or 32 code bytes and its E8M0 byte into the tile, and a
//     second barrier publishes the tile.
//   * The tile is single: the next stage's quantization starts after the
//     next stage barrier, which every wave reaches only once its reads of
//     the tile are complete.
//   * Blocks of 112 weight rows and the k order of skinny_rotation, as in
//     the kernel above for the same m: the product is bit-identical to
//     quantize-then-GEMM (mxq_quantize + mxq_gemm_w4a4, or
//     mxq_quantize_fp8 + mxq_gemm_w4a8).
template <int MT, int NW, int KS, bool RS>
struct SkDynSlot {
  using G = SkGeom<KS, false>;
  static constexpr int XRowB = 2 * KS;        // bf16 bytes per activation row
  static constexpr int XRPI = 1024 / XRowB;   // activation rows per 1-KiB copy (1 or 2)
  uint8_t w[16 * NW * G::RowB];               // weight codes
  uint8_t x[(MT + XRPI) * XRowB];             // bf16 activation rows, one copy's worth of scratch
  uint8_t ws[RS ? 16 : NW * 256];             // weight scales (256-byte region per 16 rows)
};
template <int MT, int NW, int KS, bool RS, int B>
__device__ __forceinline__ SkDynSlot<MT, NW, KS, RS>& sk_dyn_slot() {
  __shared__ __attribute__((aligned(1024))) SkDynSlot<MT, NW, KS, RS> slot;
  return slot;
}
template <int MT, int KS, bool kFp8>
struct SkDynTile {
  // codes in the layout of the activation slot above: unit v of row r at
  // slot v ^ (r % swz(units per row))
  uint8_t x[MT * SkGeom<KS, kFp8>::XRowB];
  uint8_t xs[MT / 16 * 256];   // E8M0 codes, a 256-byte region per 16 rows
};
template <int MT, int KS, bool kFp8>
__device__ __forceinline__ SkDynTile<MT, KS, kFp8>& sk_dyn_tile() {
  __shared__ __attribute__((aligned(1024))) SkDynTile<MT, KS, kFp8> tile;
  return tile;
}

template <bool kFp8, int MT, int NW, int NR, int KS, bool RS, bool kBf16Out>
__global__ __launch_bounds__(64 * NW, 1) void k_dynamic_skinny(const uint16_t* __restrict__ x,
                                                              const uint8_t* __restrict__ bq,
                                                              const uint8_t* __restrict__ bs, int64_t m,
                                                              int64_t n, int64_t k, void* __restrict__ c) {
  using G = SkGeom<KS, kFp8>;
  using Slot = SkDynSlot<MT, NW, KS, RS>;
  constexpr int RB = 16 * NW;                         // weight rows per block
  constexpr int MTT = MT / 16;                        // 16-row activation tiles
  constexpr int WC = 16 / G::RPI;                     // weight code copies per wave
  constexpr int XU = Slot::XRowB / 16;                // 16-byte units per bf16 row
  constexpr int XC = (MT / Slot::XRPI + NW - 1) / NW; // activation copies per wave
  constexpr int D = WC + (RS ? 0 : 1) + XC;           // copies per wave per stage
  constexpr int BPR = KS / 32;                        // MX blocks per row per stage
  constexpr int NB = MT * BPR;                        // MX blocks per stage
  constexpr int QPL = (NB + 64 * NW - 1) / (64 * NW); // blocks each lane quantizes
  constexpr int WSW = swz(G::U), TSW = swz(G::XU);
  static_assert(MT % 16 == 0 && NR >= 2 && NR <= 4 && (NR - 2) * D < 64, "tile / ring depth / vmcnt range");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform, as in k_gemm_skinny
  const int g = lane >> 4, col = lane & 15;
  // every wave pads its activation copies to the same count (skipping the
  // pads as k_gemm_skinny does measured within 1 % either way here)
  constexpr bool xfull = true;
  const int64_t n0 = (int64_t)blockIdx.x * RB;
  const int rows_w = (int)min((int64_t)RB, n - n0);
  const int64_t kq = k / 2, ks = k / 32, kx = 2 * k;
  const int nst = (int)(k / KS);
  const int rot = skinny_rotation<KS>(k);
  auto stage_of = [&](int s) -> unsigned {
    const int sl0 = min(s, nst - 1);
    return (unsigned)(sl0 + rot < nst ? sl0 + rot : sl0 + rot - nst);
  };
  // resident weight scale rows (k <= kSkResK), as in k_gemm_skinny
  constexpr int KSMAX = kSkResK / 32;
  constexpr int PU = KSMAX / 64;
  __shared__ __attribute__((aligned(16))) uint8_t wres[RS ? NW * 16 * (KSMAX + 16) : 16];
  const int rsp = (int)ks + 16;
  const int upr = (int)(ks >> 4);

  unsigned offw[WC], offx[XC];
  int dx[XC];
#pragma unroll
  for (int q = 0; q < WC; q++) {
    const int row = 16 * wave + G::RPI * q + lane / G::U;
    const unsigned unit = (unsigned)((lane % G::U) ^ (row % WSW));
    offw[q] = (unsigned)min(row, rows_w - 1) * (unsigned)kq + (unit << 4);
  }
  const int srow = (lane % (16 * G::LPR)) / G::LPR;
  const unsigned offws = (unsigned)min(16 * wave + srow, rows_w - 1) * (unsigned)ks + 4u * (unsigned)(lane % G::LPR);
#pragma unroll
  for (int j = 0; j < XC; j++) {
    const int a = wave + NW * j;  // copy slot (wave-uniform): activation rows XRPI a ..
    const int row = Slot::XRPI * a + lane / XU;
    offx[j] = (unsigned)min((int64_t)row, m - 1) * (unsigned)kx + ((unsigned)(lane % XU) << 4);
    dx[j] = (Slot::XRPI * a < MT ? Slot::XRPI * a : MT) * Slot::XRowB;
  }
  const __amdgpu_buffer_rsrc_t rw = panel_rsrc(bq + n0 * kq, rows_w * kq);
  const __amdgpu_buffer_rsrc_t rws = panel_rsrc(bs + n0 * ks, rows_w * ks);
  const __amdgpu_buffer_rsrc_t rx = panel_rsrc(x, m * kx);

  auto issue = [&](auto slot_tag, int s) {
    constexpr int B = decltype(slot_tag)::value;
    Slot& sl = sk_dyn_slot<MT, NW, KS, RS, B>();
    const unsigned sc = stage_of(s);
#pragma unroll
    for (int q = 0; q < WC; q++)
      bdma16_nt(rw, offw[q], sc * G::RowB, sl.w + (16 * wave + G::RPI * q) * G::RowB);
    if constexpr (!RS) bdma4(rws, offws, sc * G::ScB, sl.ws + 256 * wave);
#pragma unroll
    for (int j = 0; j < XC; j++) bdma16(rx, offx[j], sc * Slot::XRowB, sl.x + dx[j]);
  };

  SkDynTile<MT, KS, kFp8>& tile = sk_dyn_tile<MT, KS, kFp8>();
  auto quantize = [&](auto slot_tag) {
    constexpr int B = decltype(slot_tag)::value;
    const Slot& sl = sk_dyn_slot<MT, NW, KS, RS, B>();
#pragma unroll
    for (int j = 0; j < QPL; j++) {
      const int q = tid + 64 * NW * j;
      if (NB % (64 * NW) == 0 || q < NB) {
        const int r = q / BPR, b = q % BPR;
        bf16x8 xb[4];
#pragma unroll
        for (int u = 0; u < 4; u++) xb[u] = *(const bf16x8*)(sl.x + r * Slot::XRowB + (4 * b + u) * 16);
        unsigned code;
        uint8_t* trow = tile.x + r * G::XRowB;
        if constexpr (kFp8) {
          u32x2 cb[4];
          mx8_quantize_lane_bf16(xb, &code, cb);
          *(u32x4*)(trow + (((2 * b) ^ (r % TSW)) << 4)) = (u32x4){cb[0].x, cb[0].y, cb[1].x, cb[1].y};
          *(u32x4*)(trow + (((2 * b + 1) ^ (r % TSW)) << 4)) = (u32x4){cb[2].x, cb[2].y, cb[3].x, cb[3].y};
        } else {
          *(u32x4*)(trow + ((b ^ (r % TSW)) << 4)) = mx_quantize_lane_bf16(xb, &code);
        }
        tile.xs[(r / 16) * 256 + (r % 16) * G::ScB + b] = (uint8_t)code;
      }
    }
  };

  f32x4 acc[MTT];
#pragma unroll
  for (int t = 0; t < MTT; t++) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int wrow = 16 * wave + col;
  auto compute = [&](auto slot_tag, unsigned sc) {
    constexpr int B = decltype(slot_tag)::value;
    const Slot& sl = sk_dyn_slot<MT, NW, KS, RS, B>();
    unsigned wss[G::STEPS], xss[MTT][G::STEPS];
    auto words = [&](const uint8_t* p, unsigned (&wds)[G::STEPS]) {
      if constexpr (G::STEPS == 4) {
        const u32x4 v = *(const u32x4*)p;
        wds[0] = v.x; wds[1] = v.y; wds[2] = v.z; wds[3] = v.w;
      } else {
        const u32x2 v = *(const u32x2*)p;
        wds[0] = v.x; wds[1] = v.y;
      }
    };
    words(RS ? wres + wrow * rsp + sc * G::ScB : sl.ws + 256 * wave + col * G::ScB, wss);
#pragma unroll
    for (int t = 0; t < MTT; t++) words(tile.xs + 256 * t + col * G::ScB, xss[t]);
#pragma unroll
    for (int i = 0; i < G::STEPS; i++) {
      const int slot = ((4 * i + g) ^ (col % WSW)) << 4;
      const u32x4 cw = *(const u32x4*)(sl.w + wrow * G::RowB + slot);
      const i32x8 wf = {(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
      const int sw = (int)((wss[i] >> (8 * g)) & 0xFFu);
#pragma unroll
      for (int t = 0; t < MTT; t++) {
        const uint8_t* xr = tile.x + (16 * t + col) * G::XRowB;
        i32x8 xf;
        if constexpr (kFp8) {
          const u32x4 lo = *(const u32x4*)(xr + (((8 * i + g) ^ (col % TSW)) << 4));
          const u32x4 hi = *(const u32x4*)(xr + (((8 * i + 4 + g) ^ (col % TSW)) << 4));
          xf = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
          const u32x4 cx = *(const u32x4*)(xr + (((4 * i + g) ^ (col % TSW)) << 4));
          xf = (i32x8){(int)cx.x, (int)cx.y, (int)cx.z, (int)cx.w, 0, 0, 0, 0};
        }
        const int sx = (int)((xss[t][i] >> (8 * g)) & 0xFFu);
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xf, wf, acc[t], kFp8 ? kFmtFp8 : kFmtFp4, kFmtFp4,
                                                                  0, sx, 0, sw);
      }
    }
  };

  // One stage: wait for its copies and for this wave's LDS reads, meet,
  // refill, quantize the stage's activations into the tile, meet again,
  // multiply.
  auto step = [&](auto slot_tag, int s) {
    constexpr int B = decltype(slot_tag)::value;
    constexpr int N = (NR - 2) * D, N1 = (NR - 2) * (D - 1);
    if (xfull)
      __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    else
      __builtin_amdgcn_s_waitcnt((N1 & 15) | ((N1 >> 4) << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    issue(std::integral_constant<int, (B + NR - 1) % NR>{}, s + NR - 1);
    if (s < nst) {
      quantize(slot_tag);
      __builtin_amdgcn_s_waitcnt((15 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      compute(slot_tag, stage_of(s));
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1 % NR>;
  using I2 = std::integral_constant<int, 2 % NR>;
  using I3 = std::integral_constant<int, 3 % NR>;
  u32x4 wsv[RS ? PU : 1];
  if constexpr (RS) {
#pragma unroll
    for (int p = 0; p < PU; p++) {
      const int i = lane + 64 * p;
      const int r = i / upr, cu = i - r * upr;
      const int row = min(16 * wave + min(r, 15), rows_w - 1);
      wsv[p] = *(const u32x4*)(bs + (n0 + row) * ks + 16 * cu);
    }
  }
  issue(I0{}, 0);
  if (NR > 2) issue(I1{}, 1);
  if (NR > 3) issue(I2{}, 2);
  if constexpr (RS) {
    // older than the NR - 1 stages of copies in flight; only this wave
    // reads its rows' scales
    if (xfull)
      wait_vmcnt<(NR - 1) * D>();
    else
      wait_vmcnt<(NR - 1) * (D - 1)>();
#pragma unroll
    for (int p = 0; p < PU; p++) {
      const int i = lane + 64 * p;
      const int r = i / upr, cu = i - r * upr;
      if (r < 16) *(u32x4*)(wres + (16 * wave + r) * rsp + 16 * cu) = wsv[p];
    }
  }
  step(I0{}, 0);
  for (int s = 1; s < nst; s += NR) {
    step(I1{}, s);
    if (NR > 2) step(I2{}, s + 1);
    if (NR > 3) step(I3{}, s + 2);
    step(I0{}, s + NR - 1);
  }
  wait_vmcnt<0>();

  const int64_t nn = n0 + wrow;
  if (nn < n) {
#pragma unroll
    for (int t = 0; t < MTT; t++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int64_t mm = 16 * t + 4 * g + e;
        if (mm >= m) continue;
        if (kBf16Out)
          ((uint16_t*)c)[mm * n + nn] = f32_to_bf16_rne(acc[t][e]);
        else
          ((float*)c)[mm * n + nn] = acc[t][e];
      }
  }
}

// Launch configurations <MT, NW, NR, KS> per activation tile.  The LDS
// ring holds at most 160 KiB: the 128-row tile of E2M1 activations fits
// two 512-k stages, the 64- and 128-row E4M3 tiles take 256-k stages.
#ifndef MXQ_SK4_C16
#define MXQ_SK4_C16 16, 7, 3, 512
#endif
#ifndef MXQ_SK4_C32
#define MXQ_SK4_C32 32, 7, 3, 512
#endif
#ifndef MXQ_SK4_C64
#define MXQ_SK4_C64 64, 7, 3, 512
#endif
#ifndef MXQ_SK4_C128
#define MXQ_SK4_C128 128, 7, 2, 512
#endif
#ifndef MXQ_SK8_C16
#define MXQ_SK8_C16 16, 7, 3, 512
#endif
#ifndef MXQ_SK8_C32
#define MXQ_SK8_C32 32, 7, 3, 512
#endif
#ifndef MXQ_SK8_C64
#define MXQ_SK8_C64 64, 7, 4, 256
#endif
#ifndef MXQ_SK8_C128
#define MXQ_SK8_C128 128, 7, 3, 256
#endif

bool gemm_skinny_applies(int64_t m, int64_t k) {
  // 32-bit copy offsets: a weight panel of at most 224 rows and a 128-row
  // activation panel stay below 2^31 bytes for k <= 2^24
  return m >= 1 && m <= 128 && k >= 512 && k % 512 == 0 && k <= (1 << 24);
}

// Up to 16 activation rows with k <= kSkResK: resident scale rows, 256-k
// stages in a 4-slot ring.  Measured on a 28672 x 8192 weight, m = 16
// (interleaved A/B): W4A4 21.8 us against 22.4 us with per-stage scale
// copies (512-k, 3 slots) and 21.9 us resident with 512-k stages; W4A8 21.9
// against 23.3 and 22.1 us.
#ifndef MXQ_SK_RS
#define MXQ_SK_RS 1
#endif
#ifndef MXQ_SK4_RS16
#define MXQ_SK4_RS16 16, 7, 4, 256
#endif
#ifndef MXQ_SK8_RS16
#define MXQ_SK8_RS16 16, 7, 4, 256
#endif

hipError_t launch_w4a4_skinny(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                              int64_t m, int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st) {
  if (m <= 16 && MXQ_SK_RS && k <= kSkResK)
    launch_sk<false, MXQ_SK4_RS16, true>(aq, as, bq, bs, m, n, k, c, bf16_out, st);
  else if (m <= 16)
    launch_sk<false, MXQ_SK4_C16>(aq, as, bq, bs, m, n, k, c, bf16_out, st);
  else if (m <= 32)
    launch_sk<false, MXQ_SK4_C32>(aq, as, bq, bs, m, n, k, c, bf16_out, st);
  else if (m <= 64)
    launch_sk<false, MXQ_SK4_C64>(aq, as, bq, bs, m, n, k, c, bf16_out, st);
  else
    launch_sk<false, MXQ_SK4_C128>(aq, as, bq, bs, m, n, k, c, bf16_out, st);
  return hipGetLastError();
}

hipError_t launch_w4a8_skinny(const uint8_t* aq8, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                              int64_t m, int64_t n, int64_t k, void* c, bool bf16_out, hipStream_t st) {
  if (m <= 16 && MXQ_SK_RS && k <= kSkResK)
    launch_sk<true, MXQ_SK8_RS16, true>(aq8, as, bq, bs, m, n, k, c, bf16_out, st);
  else if (m <= 16)
    launch_sk<true, MXQ_SK8_C16>(aq8, as, bq, bs, m, n, k, c, bf16_out, st);
  else if (m <= 32)
    launch_sk<true, MXQ_SK8_C32>(aq8, as, bq, bs, m, n, k, c, bf16_out, st);
  else if (m <= 64)
    launch_sk<true, MXQ_SK8_C64>(aq8, as, bq, bs, m, n, k, c, bf16_out, st);
  else
    launch_sk<true, MXQ_SK8_C128>(aq8, as, bq, bs, m, n, k, c, bf16_out, st);
  return hipGetLastError();
}

template <bool kFp8, int MT, int NW, int NR, int KS, bool RS = false>
static void launch_skd(const uint16_t* x, const uint8_t* bq, const uint8_t* bs, int64_t m, int64_t n, int64_t k,
                       void* c, bool bf16_out, hipStream_t st) {
  const dim3 grid((unsigned)((n + 16 * NW - 1) / (16 * NW)));
  if (bf16_out)
    hipLaunchKernelGGL((k_dynamic_skinny<kFp8, MT, NW, NR, KS, RS, true>), grid, dim3(64 * NW), 0, st, x, bq, bs, m,
                       n, k, c);
  else
    hipLaunchKernelGGL((k_dynamic_skinny<kFp8, MT, NW, NR, KS, RS, false>), grid, dim3(64 * NW), 0, st, x, bq, bs,
                       m, n, k, c);
}

// Up to 16 activation rows.  Measured on a 28672 x 8192 weight against
// quantize + the product kernel: W4A4 22.7 vs 24.5-24.8 us at m = 1,
// 25.1-25.7 vs 24.9 us at m = 16, but 33.5 vs 27.2 us at m = 32 and 50.6 vs
// 29.9 us at m = 64; W4A8 23.6 vs 25.1-25.5 us at m = 1, 26.4-27.6 vs 26.4 us
// at m = 16, 38.6-42.0 vs 29.2-29.6 us at m = 32.  Every block pulls a
// bf16 tile (4x the bytes of MXFP4 codes, 2x those of MXFP8) through the
// same copy path as the weights.
// W4A4, k <= kSkResK: resident weight scale rows, 256-k stages in 4 slots
// (m = 16 on a 28672 x 8192 weight: 23.2-23.5 against 24.9 us).  The same
// shape made W4A8 slower (26.3 against 24.8 us), which keeps 512-k stages
// with per-stage scale copies.
#ifndef MXQ_SKD_RS16
#define MXQ_SKD_RS16 16, 7, 4, 256
#endif
hipError_t launch_w4a4_dynamic(const uint16_t* x, const uint8_t* bq, const uint8_t* bs, int64_t m, int64_t n,
                               int64_t k, void* c, bool bf16_out, hipStream_t st) {
  if (MXQ_SK_RS && k <= kSkResK)
    launch_skd<false, MXQ_SKD_RS16, true>(x, bq, bs, m, n, k, c, bf16_out, st);
  else
    launch_skd<false, 16, 7, 3, 512>(x, bq, bs, m, n, k, c, bf16_out, st);
  return hipGetLastError();
}

hipError_t launch_w4a8_dynamic(const uint16_t* x, const uint8_t* bq, const uint8_t* bs, int64_t m, int64_t n,
                               int64_t k, void* c, bool bf16_out, hipStream_t st) {
  launch_skd<true, 16, 7, 3, 512>(x, bq, bs, m, n, k, c, bf16_out, st);
  return hipGetLastError();
}

}  // namespace mxq
