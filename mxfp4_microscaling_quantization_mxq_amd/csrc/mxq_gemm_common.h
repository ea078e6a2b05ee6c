// mxq_gemm_common.h -- device helpers shared by the product kernels (W4A4,
// W4A8, W4A16 and the small-m kernels): direct global / buffer -> LDS
// copies, wait counts and scheduling hints, and the LDS-staged epilogue
// stores.
#pragma once
#include "mxq_device.h"

namespace mxq {

// Output kinds of the product kernels: fp32, bf16, or MXFP4 (the bf16-rounded
// product quantized along n, bit-identical to mxq_quantize of the bf16
// output: the quantizer is the same device function).
constexpr int kOutF32 = 0, kOutBf16 = 1, kOutMx = 2;

// Operand format codes of the f8f6f4 block-scaled MFMA (E4M3, E2M1).
constexpr int kFmtFp8 = 0, kFmtFp4 = 4;

// Quantizes a bf16 output tile staged in LDS and stores its codes and E8M0
// scales.  The tile has ROWS rows of COLS bytes (COLS / 16 units of 8 bf16);
// rows [0, 128) sit in lo and [128, ROWS) in hi (two LDS variables when the
// tile exceeds one), row r at (r % 128) * COLS bytes of its region, unit u
// of row r at u ^ (r % (COLS / 16)).
// Four consecutive threads take the four units (32 columns) of one MXFP4
// block; blocks past m or n are computed but not stored (n % 32 == 0).
template <int ROWS, int COLS>
__device__ __forceinline__ void store_mx_tile(const uint8_t* lo, const uint8_t* hi, int64_t m0, int64_t n0,
                                              int64_t m, int64_t n, uint8_t* __restrict__ cq,
                                              uint8_t* __restrict__ cs) {
  constexpr int UNITS = COLS / 16;  // 16-byte units (8 bf16) per row
  for (int u = threadIdx.x; u < ROWS * UNITS; u += blockDim.x) {
    const int r = u / UNITS, unit = u % UNITS;
    const uint8_t* base = r < 128 ? lo : hi;
    const bf16x8 xb = *(const bf16x8*)(base + (r & 127) * COLS + ((unit ^ (r % UNITS)) << 4));
    unsigned code;
    const unsigned codes = mx_quantize_quad_bf16(xb, &code);
    const int64_t gr = m0 + r, gc = n0 + 8 * unit;
    if (gr < m && gc < n) {
      *(unsigned*)(cq + gr * (n / 2) + gc / 2) = codes;
      if ((unit & 3) == 0) cs[gr * (n / 32) + gc / 32] = (uint8_t)code;
    }
  }
}

// Stores a bf16 output tile staged in LDS (layout as in store_mx_tile) in
// whole 16-byte units: consecutive threads write consecutive units of a
// row.  A unit that crosses n (n % 8 != 0) is stored element by element.
template <int ROWS, int COLS>
__device__ __forceinline__ void store_bf16_tile(const uint8_t* lo, const uint8_t* hi, int64_t m0, int64_t n0,
                                                int64_t m, int64_t n, uint16_t* __restrict__ c) {
  constexpr int UNITS = COLS / 16;
  for (int u = threadIdx.x; u < ROWS * UNITS; u += blockDim.x) {
    const int r = u / UNITS, unit = u % UNITS;
    const uint8_t* base = r < 128 ? lo : hi;
    const u32x4 v = *(const u32x4*)(base + (r & 127) * COLS + ((unit ^ (r % UNITS)) << 4));
    const int64_t gr = m0 + r, gc = n0 + 8 * unit;
    if (gr >= m || gc >= n) continue;
    uint16_t* dst = c + gr * n + gc;
    if (gc + 8 <= n && (n & 7) == 0) {
      *(u32x4*)dst = v;
    } else {
      const unsigned w[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 8 && gc + e < n; e++) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
// The same 16-byte copy through a buffer resource (buffer_load_dwordx4 ...
// lds): base and size in SGPRs, a 32-bit per-lane offset and a uniform
// offset; reads past the size return zero.  Measured about 3 % faster than
// the 64-bit-address form in the block-scaled GEMM rings.  The compiler
// tracks it as a plain vector-memory load, not as an LDS write: the kernels
// wait for it with explicit vmcnt counts before a barrier.
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3
__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)voff, (int)soff, 0, 0);
}
// Streaming form for operands every block reads exactly once (the decode
// weight): cache-policy operand 2 sets the non-temporal bit ("nt" in the
// instruction).  On a 28672 x 8192 decode weight the hint took the m = 4
// ring from 24.1 to 22.5 us.
__device__ __forceinline__ void bdma16_nt(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)voff, (int)soff, 0, 2);
}
// 4-byte form: the copy places one dword per lane (LDS base + 4 i).
__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}
// s_waitcnt vmcnt(n) with every other counter left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Scheduling hint: R LDS reads, then MG MFMAs, four times over.
template <int R, int MG = 4>
__device__ __forceinline__ void interleave_reads_mfma() {
#pragma unroll
  for (int g = 0; g < 4; g++) {
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MG, 0);
  }
}

}  // namespace mxq
