// quant.hip -- MXFP4 and NVFP4 quantize / dequantize kernels (gfx950).
//
// Memory-bound elementwise work: every kernel streams its input once with
// 16-byte loads per lane (1 KiB per wave instruction, fully coalesced) and
// writes packed codes with 4-byte stores per lane (256 contiguous bytes per
// wave).  The element conversion uses the CDNA4 scaled-convert
// instructions, whose rounding (to nearest even), saturation (+-6), signed
// zeros and subnormal handling were checked bit-exact against the CPU
// oracle over every bf16 pattern and every E8M0 scale.
//
// Method [TransFP4 page "Portable FP4 quantization for heterogeneous
// accelerators", sec. 1.1 eq. (1)]: x_hat = s_g * s_b * Q(x / (s_g * s_b)).
#include "mxq_device.h"
#include "mxq_launch.h"

namespace mxq {

// Output stores of the streaming kernels: every byte is written once and not
// read again by the kernel, so they carry the streaming hint
// (MXQ_NT_STORE 1) or are plain stores (0).  Interleaved A/B, 16384 x 8192:
// MXFP4 dequantize to bf16 61.2-61.7 -> 49.1 us, NVFP4 61.5-61.7 -> 49.7,
// TransFP4 71.2 -> 67.7, the NVFP4 quantize pass (4096 x 8192) 30.0 -> 29.2,
// the MXFP4 quantizer even.  The MXFP8 and rotated MXFP4 quantizers measured
// 1 % faster with plain stores and keep them.  (The same hint on the tiled
// GEMMs' output stores, which write each row of a tile in pieces, cost
// 28 % on the 4096 x 8192 x 4096 W4A16 GEMM.)
#ifndef MXQ_NT_STORE
#define MXQ_NT_STORE 1
#endif
template <class T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  if constexpr (MXQ_NT_STORE)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// ---------------------------------------------------------------- MXFP4

// One lane = 8 consecutive elements; a quad of lanes = one 32-element block
// [infra-guide "4.5 FP8 and NVFP4/MXFP4", sec. 4.1: 32 E2M1 + one E8M0].
// The block absmax is an integer max over magnitude bits, shared inside the
// quad with two DPP steps; the E8M0 exponent floor(log2 amax) - 2 is read
// straight off the exponent field.
// A block takes kQuantU chunks of 256 lanes and issues all their loads
// before any arithmetic (more bytes in flight per wave); lanes past the end
// re-read the first chunk's lane and store nothing.  nlanes is a multiple
// of 4 and chunks are 256 lanes, so quads stay whole.
// Chunks per block, measured (interleaved A/B against one chunk per block)
// on the dynamic-quantize tensor 16384 x 8192 bf16 and an 8192 x 8192 one:
// MXFP4 54.9 -> 52.4 us with 2 (53.2 with 4); MXFP8 35.7 -> 32.8 us with 4
// (33.3 with 2); rotated MXFP4 (hk 32) 61.9 -> 52.7 us with 4 (55.2 with
// 2); NVFP4 quantize pass of the 8192 x 4096 weight: 31.7 -> 30.9 us.
#ifndef MXQ_QUANT_U
#define MXQ_QUANT_U 2
#endif
#ifndef MXQ_QUANT8_U
#define MXQ_QUANT8_U 4
#endif
#ifndef MXQ_HAD_U
#define MXQ_HAD_U 4
#endif
#ifndef MXQ_NVQ_U
#define MXQ_NVQ_U 2
#endif
constexpr int kQuantU = MXQ_QUANT_U, kQuant8U = MXQ_QUANT8_U, kHadU = MXQ_HAD_U, kNvqU = MXQ_NVQ_U;
__global__ __launch_bounds__(256) void k_mx_quantize_bf16(const u32x4* __restrict__ x,
                                                          unsigned* __restrict__ q,
                                                          uint8_t* __restrict__ s,
                                                          int64_t nlanes) {
  const int64_t t0 = (int64_t)blockIdx.x * (256 * kQuantU) + threadIdx.x;
  if (t0 >= nlanes) return;
  bf16x8 xb[kQuantU];
#pragma unroll
  for (int u = 0; u < kQuantU; u++) {
    const int64_t t = t0 + 256 * u;
    xb[u] = __builtin_nontemporal_load((const bf16x8*)&x[t < nlanes ? t : t0]);
  }
#pragma unroll
  for (int u = 0; u < kQuantU; u++) {
    const int64_t t = t0 + 256 * u;
    unsigned code;
    const unsigned out = mx_quantize_quad_bf16(xb[u], &code);
    if (t < nlanes) {
      st_stream(&q[t], out);
      if ((t & 3) == 0) s[t >> 2] = (uint8_t)code;
    }
  }
}

__global__ __launch_bounds__(256) void k_mx_quantize_f32(const u32x4* __restrict__ x,
                                                         unsigned* __restrict__ q,
                                                         uint8_t* __restrict__ s,
                                                         int64_t nlanes) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nlanes) return;
  u32x4 a = __builtin_nontemporal_load(&x[2 * t]);
  u32x4 b = __builtin_nontemporal_load(&x[2 * t + 1]);
  unsigned m = max(max(max(a.x & 0x7FFFFFFFu, a.y & 0x7FFFFFFFu), max(a.z & 0x7FFFFFFFu, a.w & 0x7FFFFFFFu)),
                   max(max(b.x & 0x7FFFFFFFu, b.y & 0x7FFFFFFFu), max(b.z & 0x7FFFFFFFu, b.w & 0x7FFFFFFFu)));
  m = max(m, dpp_quad_xor1(m));
  m = max(m, dpp_quad_xor2(m));
  unsigned code = e8m0_code_from_expfield(m >> 23);
  float scale = e8m0_as_scale(code);
  unsigned out = 0;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(a.x), __uint_as_float(a.y), scale, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(a.z), __uint_as_float(a.w), scale, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(b.x), __uint_as_float(b.y), scale, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(b.z), __uint_as_float(b.w), scale, 3);
  st_stream(&q[t], out);
  if ((t & 3) == 0) s[t >> 2] = (uint8_t)code;
}

// Dequantize: one lane = 4 code bytes = 8 elements, scale byte t/4.
// kDeqU chunks of 256 lanes per block with every load issued first (a
// lane's own loads are 4 code bytes and a scale byte: one chunk per thread
// left the loads' latency exposed).  16384 x 8192 to bf16: MXFP4 62.3 ->
// 60.2 us, NVFP4 83.8 -> 60.1 us (8 chunks: 63.7 and 65.3 us).
#ifndef MXQ_DEQ_U
#define MXQ_DEQ_U 4
#endif
constexpr int kDeqU = MXQ_DEQ_U;
template <bool kBf16Out>
__global__ __launch_bounds__(256) void k_mx_dequantize(const unsigned* __restrict__ q,
                                                       const uint8_t* __restrict__ s,
                                                       void* __restrict__ y, int64_t nlanes) {
  const int64_t t0 = (int64_t)blockIdx.x * (256 * kDeqU) + threadIdx.x;
  if (t0 >= nlanes) return;
  unsigned cv[kDeqU], sv[kDeqU];
#pragma unroll
  for (int u = 0; u < kDeqU; u++) {
    const int64_t t = t0 + 256 * u < nlanes ? t0 + 256 * u : t0;
    cv[u] = q[t];
    sv[u] = s[t >> 2];
  }
#pragma unroll
  for (int u = 0; u < kDeqU; u++) {
    const int64_t t = t0 + 256 * u;
    if (t >= nlanes) break;
    const unsigned c = cv[u];
    const float scale = e8m0_as_scale(sv[u]);
    if (kBf16Out) {
      u32x4 o;
      o.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0));
      o.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1));
      o.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2));
      o.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3));
      st_stream(&((u32x4*)y)[t], o);
    } else {
      auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 0);
      auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 1);
      auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 2);
      auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, scale, 3);
      f32x4 o0 = {p0[0], p0[1], p1[0], p1[1]};
      f32x4 o1 = {p2[0], p2[1], p3[0], p3[1]};
      st_stream(&((f32x4*)y)[2 * t], o0);
      st_stream(&((f32x4*)y)[2 * t + 1], o1);
    }
  }
}

// ---------------------------------------------------------------- MXFP8

// MXFP8: E4M3 elements with one E8M0 scale per 32 [infra-guide "4.5 FP8 and
// NVFP4/MXFP4", sec. 4.2: the mxfp8 scheme, FP8 values and an E8M0 scale
// per 1x32; sec. 1.2: E4M3, max 448, NaN only].  Block exponent by the
// MXFP4 rule with E4M3's top exponent: code = max(expfield(amax) - 8, 0),
// i.e. floor(log2 amax) - 8 + 127, so the block's largest magnitude scales
// into [256, 512).  Elements: the gfx950 scaled fp8 convert (round to
// nearest even), after clamping every magnitude to 448 * 2^e: the convert
// itself turns scaled values past 448 into the NaN code instead of
// saturating (seen in the bit-exact comparison with the CPU oracle), and the
// clamp is exact (448 * 2^e is a bf16 / fp32 number, and x * 2^-e is exact).
// One lane = 8 elements, a quad = one block; a lane stores 8 code bytes.
typedef short s16x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void k_mx8_quantize_bf16(const u32x4* __restrict__ x, u32x2* __restrict__ q,
                                                           uint8_t* __restrict__ s, int64_t nlanes) {
  // kQuant8U chunks of 256 lanes per block, loads first (as k_mx_quantize_bf16)
  const int64_t t0 = (int64_t)blockIdx.x * (256 * kQuant8U) + threadIdx.x;
  if (t0 >= nlanes) return;  // quads stay whole
  bf16x8 xb[kQuant8U];
#pragma unroll
  for (int u = 0; u < kQuant8U; u++) {
    const int64_t t = t0 + 256 * u;
    xb[u] = __builtin_nontemporal_load((const bf16x8*)&x[t < nlanes ? t : t0]);
  }
#pragma unroll
  for (int u = 0; u < kQuant8U; u++) {
    const int64_t t = t0 + 256 * u;
    unsigned m = bf16x8_absmax_bits(xb[u]);
    m = max(m, dpp_quad_xor1(m));
    m = max(m, dpp_quad_xor2(m));
    const unsigned code = e8m0_code_e4m3(m >> 7);
    const u32x2 out = mx8_encode8_bf16(xb[u], code);
    if (t < nlanes) {
      q[t] = out;
      if ((t & 3) == 0) s[t >> 2] = (uint8_t)code;
    }
  }
}

__global__ __launch_bounds__(256) void k_mx8_quantize_f32(const u32x4* __restrict__ x, u32x2* __restrict__ q,
                                                          uint8_t* __restrict__ s, int64_t nlanes) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nlanes) return;
  const u32x4 a = __builtin_nontemporal_load(&x[2 * t]);
  const u32x4 b = __builtin_nontemporal_load(&x[2 * t + 1]);
  unsigned m = max(max(max(a.x & 0x7FFFFFFFu, a.y & 0x7FFFFFFFu), max(a.z & 0x7FFFFFFFu, a.w & 0x7FFFFFFFu)),
                   max(max(b.x & 0x7FFFFFFFu, b.y & 0x7FFFFFFFu), max(b.z & 0x7FFFFFFFu, b.w & 0x7FFFFFFFu)));
  m = max(m, dpp_quad_xor1(m));
  m = max(m, dpp_quad_xor2(m));
  const unsigned code = e8m0_code_e4m3(m >> 23);
  const float scale = e8m0_as_scale(code);
  // |x| clamped to 448 * 2^e (fp32 bits: exponent field code + 8, mantissa .11)
  const unsigned lim = ((code + 8u) << 23) | 0x600000u;
  auto clamp = [&](unsigned w) { return __uint_as_float(min(w & 0x7FFFFFFFu, lim) | (w & 0x80000000u)); };
  s16x2 lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, clamp(a.x), clamp(a.y), scale, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, clamp(a.z), clamp(a.w), scale, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, clamp(b.x), clamp(b.y), scale, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, clamp(b.z), clamp(b.w), scale, true);
  q[t] = (u32x2){__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
  if ((t & 3) == 0) s[t >> 2] = (uint8_t)code;
}

// ---------------------------------------------------------------- rotated MXFP4

// Block Hadamard rotation fused ahead of the MXFP4 quantizer: y_j = H x_j
// per block of HK elements along k, H the Sylvester-ordered Hadamard matrix
// divided by sqrt(HK) (orthonormal, so the error can be judged in the
// rotated domain [TransFP4 page sec. 2.3 eq. (2)]; the activation side
// computes X H_k online with a butterfly network, k in {16, 32, 64, 128}
// ["FP4 quantization analysis" page, sec. 3.2.3]).  In fp32 the rotation
// rounds, so its order of operations is fixed: butterfly stages h = 1, 2,
// 4, ..., HK/2 over pairs (i, i + h), (u, v) -> (u + v, u - v), then one
// multiply by the fp32 nearest 1/sqrt(HK).  A lane holds 8 consecutive
// elements: stages h < 8 run inside the lane, h = 8 m between lanes l and
// l ^ m (the lane with bit m clear keeps the sum, the other partner - own =
// u - v).  The rotated fp32 values then go through the fp32 MXFP4 path.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (M == 1)
    return __uint_as_float(dpp_quad_xor1(__float_as_uint(v)));
  else if constexpr (M == 2)
    return __uint_as_float(dpp_quad_xor2(__float_as_uint(v)));
  else if constexpr (M == 4)
    return __shfl_xor(v, 4, 64);
  else  // row_ror:8 inside a row of 16 lanes: lane l ^ 8
    return __uint_as_float((unsigned)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x128, 0xF, 0xF, false));
}

template <int HK>
__device__ __forceinline__ float hadamard_norm() {
  // 1/sqrt(16) and 1/sqrt(64) are exact; for 32 and 128 the fp32 nearest
  // 1/sqrt(2) (0x3F3504F3) divided exactly by 4 and by 8
  if constexpr (HK == 16) return 0.25f;
  else if constexpr (HK == 32) return 0x1.6a09e6p-3f;
  else if constexpr (HK == 64) return 0.125f;
  else return 0x1.6a09e6p-4f;
}

template <int M>
__device__ __forceinline__ void butterfly_across_lanes(float (&v)[8], int lane) {
  const bool upper = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float p = lane_xor<M>(v[i]);
    v[i] = upper ? p - v[i] : v[i] + p;
  }
}

// One lane's 8 consecutive elements (lane t of the tensor) as fp32.
template <bool kBf16In>
__device__ __forceinline__ void load8(const u32x4* __restrict__ x, int64_t t, float (&v)[8]) {
  if (kBf16In) {
    const u32x4 w = __builtin_nontemporal_load(&x[t]);
    const unsigned ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(ww[i] << 16);
      v[2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
    }
  } else {
    const u32x4 a = __builtin_nontemporal_load(&x[2 * t]);
    const u32x4 b = __builtin_nontemporal_load(&x[2 * t + 1]);
    const unsigned ww[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = __uint_as_float(ww[i]);
  }
}

// H_HK applied to the HK-block that this lane's 8 values belong to (HK / 8
// consecutive lanes), in the fixed order described above.
template <int HK>
__device__ __forceinline__ void rotate8(float (&v)[8], int lane) {
  // stages h = 1, 2, 4 inside the lane
#pragma unroll
  for (int h = 1; h < 8; h *= 2)
#pragma unroll
    for (int i = 0; i < 8; i++)
      if ((i & h) == 0) {
        const float u = v[i], w = v[i + h];
        v[i] = u + w;
        v[i + h] = u - w;
      }
  // stages h = 8, 16, 32, 64 across lanes 1, 2, 4, 8 apart
  if constexpr (HK > 8) butterfly_across_lanes<1>(v, lane);
  if constexpr (HK > 16) butterfly_across_lanes<2>(v, lane);
  if constexpr (HK > 32) butterfly_across_lanes<4>(v, lane);
  if constexpr (HK > 64) butterfly_across_lanes<8>(v, lane);
  const float c = hadamard_norm<HK>();
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = v[i] * c;
}

template <bool kBf16In, int HK>
__global__ __launch_bounds__(256) void k_mx_quantize_hadamard(const u32x4* __restrict__ x, unsigned* __restrict__ q,
                                                              uint8_t* __restrict__ s, int64_t nlanes) {
  static_assert(HK == 16 || HK == 32 || HK == 64 || HK == 128, "rotation size");
  // kHadU chunks of 256 lanes per block, loads first (as k_mx_quantize_bf16).
  // nlanes is a multiple of HK / 8 and of 4, and chunks hold 256 lanes:
  // rotation groups and MXFP4 quads are whole, valid or past the end
  const int64_t t0 = (int64_t)blockIdx.x * (256 * kHadU) + threadIdx.x;
  if (t0 >= nlanes) return;
  const int lane = threadIdx.x & 63;
  float v[kHadU][8];
#pragma unroll
  for (int u = 0; u < kHadU; u++) {
    const int64_t t = t0 + 256 * u;
    load8<kBf16In>(x, t < nlanes ? t : t0, v[u]);
  }
#pragma unroll
  for (int u = 0; u < kHadU; u++) {
    const int64_t t = t0 + 256 * u;
    rotate8<HK>(v[u], lane);
    // MXFP4 of the rotated block (as k_mx_quantize_f32)
    unsigned m = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) m = max(m, __float_as_uint(v[u][i]) & 0x7FFFFFFFu);
    m = max(m, dpp_quad_xor1(m));
    m = max(m, dpp_quad_xor2(m));
    const unsigned code = e8m0_code_from_expfield(m >> 23);
    const float scale = e8m0_as_scale(code);
    unsigned out = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[u][0], v[u][1], scale, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[u][2], v[u][3], scale, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[u][4], v[u][5], scale, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[u][6], v[u][7], scale, 3);
    if (t < nlanes) {
      q[t] = out;
      if ((t & 3) == 0) s[t >> 2] = (uint8_t)code;
    }
  }
}

// ---------------------------------------------------------------- NVFP4

// Tensor amax [infra-guide sec. 2: s = max|x| / F_max], in two steps with
// no atomics: every block of k_nv_amax writes the largest magnitude of its
// grid-stride share (as fp32 bits; non-negative floats order like their
// bits) to part[block], then one block of k_nv_scale folds the partials and
// writes s_t.  part is the caller's code buffer, which the quantize pass
// overwrites afterwards in stream order.  (One same-address device-scope
// atomic per block cost about 8 us per call here: those atomics serialize
// at the memory side.)
constexpr int kAmaxU = 8;  // 16-byte loads in flight per lane

template <bool kBf16In>
__global__ __launch_bounds__(256) void k_nv_amax(const u32x4* __restrict__ x, int64_t nvec,
                                                 unsigned* __restrict__ part) {
  __shared__ unsigned wmax[4];
  unsigned m = 0;
  const int64_t stride = (int64_t)gridDim.x * 256 * kAmaxU;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kAmaxU + threadIdx.x; base - threadIdx.x < nvec;
       base += stride) {
    u32x4 v[kAmaxU];
#pragma unroll
    for (int u = 0; u < kAmaxU; u++) {
      const int64_t i = base + u * 256;
      v[u] = i < nvec ? __builtin_nontemporal_load(&x[i]) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kAmaxU; u++) {
      if (kBf16In) {
        unsigned h = bf16x2_absmax_bits(bf16x2_absmax_bits(v[u].x, v[u].y), bf16x2_absmax_bits(v[u].z, v[u].w));
        m = max(m, max(h & 0xFFFFu, h >> 16) << 16);  // as fp32 bits
      } else {
        m = max(m, max(max(v[u].x & 0x7FFFFFFFu, v[u].y & 0x7FFFFFFFu),
                       max(v[u].z & 0x7FFFFFFFu, v[u].w & 0x7FFFFFFFu)));
      }
    }
  }
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

// s_t from the tensor amax: fl32(amax / 2688), or 1 for an all-zero tensor.
__device__ __forceinline__ float nv_tensor_scale(float amax) {
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 2688.0f);
}

// One block: the largest of np partials, turned into s_t at *g.
// One block of 1024 threads; np <= 2048 partials, so every thread issues its
// (at most two) loads at once instead of a chain of dependent ones (256
// threads walking 2048 partials took about 3.6 us).
constexpr int kScaleThreads = 1024, kScaleMaxParts = 2 * kScaleThreads;
__global__ __launch_bounds__(kScaleThreads) void k_nv_scale(const unsigned* __restrict__ part, int np,
                                                            float* __restrict__ g) {
  __shared__ unsigned wmax[kScaleThreads / 64];
  const int t = threadIdx.x;
  const unsigned a = t < np ? part[t] : 0u;
  const unsigned b = t + kScaleThreads < np ? part[t + kScaleThreads] : 0u;
  unsigned m = max(a, b);
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    unsigned r = 0;
    for (int w = 0; w < kScaleThreads / 64; w++) r = max(r, wmax[w]);
    *g = nv_tensor_scale(__uint_as_float(r));
  }
}

// |x| / d rounded to nearest even (fp32), for d >= 2^-100 and |x| / d <= 2^100:
// y = RN(1/d) (one IEEE division per block), q0 = RN(|x| y), then two
// residual corrections r = |x| - d q (exact with an fma) and q += r y.
// After the first correction q is within one ulp of |x| / d; with y
// correctly rounded, the second correction returns the correctly rounded
// quotient (Markstein's theorem on fma-based division).  Quotients below
// 2^-3 may come out inexact, but every one of them still encodes to code 0.
__device__ __forceinline__ float div_by_block_scale(float ax, float d, float y) {
  float q = ax * y;
  float r = __builtin_fmaf(-d, q, ax);
  q = __builtin_fmaf(r, y, q);
  r = __builtin_fmaf(-d, q, ax);
  return __builtin_fmaf(r, y, q);
}

// One lane = 8 consecutive elements, a pair of lanes = one 16-element block
// [infra-guide sec. 4.1: 16 E2M1 + one E4M3, times the FP32 tensor scale].
// fp32 order: t = fl(6 s_t); s_b = E4M3(fl(amax_b / t));
// d = fl(s_t * s_b); q_i = E2M1_rne(fl(x_i / d)), the quotient rounded once.
template <bool kBf16In>
__global__ __launch_bounds__(256) void k_nv_quantize(const u32x4* __restrict__ x, const float* __restrict__ g,
                                                     unsigned* __restrict__ q, uint8_t* __restrict__ s,
                                                     int64_t nlanes) {
  // kNvqU chunks of 256 lanes per block, loads first (as k_mx_quantize_bf16);
  // nlanes is even and chunks hold 256 lanes: pairs stay whole
  const int64_t t0 = (int64_t)blockIdx.x * (256 * kNvqU) + threadIdx.x;
  if (t0 >= nlanes) return;
  const float st = *g;
  float xv[kNvqU][8];
#pragma unroll
  for (int u = 0; u < kNvqU; u++) {
    const int64_t t = t0 + 256 * u;
    load8<kBf16In>(x, t < nlanes ? t : t0, xv[u]);
  }
#pragma unroll
  for (int u = 0; u < kNvqU; u++) {
    const int64_t t = t0 + 256 * u;
    const float (&xs)[8] = xv[u];
    unsigned m = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) m = max(m, __float_as_uint(xs[i]) & 0x7FFFFFFFu);
    m = max(m, dpp_quad_xor1(m));
    float tden = 6.0f * st;
    unsigned sb = e4m3_encode_nonneg(__fdiv_rn(__uint_as_float(m), tden));
    float sbv = e4m3_value(sb);
    unsigned out = 0;
    if (sbv == 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; i++) out |= (__float_as_uint(xs[i]) >> 31) << (3 + 4 * i);
    } else {
      const float d = st * sbv;
      float v[8];
      if (d >= 0x1p-100f && __uint_as_float(m) <= d * 0x1p100f) {
        const float y = __fdiv_rn(1.0f, d);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const unsigned xb = __float_as_uint(xs[i]);
          const float aq = div_by_block_scale(__uint_as_float(xb & 0x7FFFFFFFu), d, y);
          v[i] = __uint_as_float(__float_as_uint(aq) | (xb & 0x80000000u));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = __fdiv_rn(xs[i], d);
      }
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[0], v[1], 1.0f, 0);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[2], v[3], 1.0f, 1);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[4], v[5], 1.0f, 2);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[6], v[7], 1.0f, 3);
    }
    if (t < nlanes) {
      st_stream(&q[t], out);
      if ((t & 1) == 0) s[t >> 1] = (uint8_t)sb;
    }
  }
}

// NVFP4 dequantize: y = s_t * (s_b * q).  s_b * q is exact in fp32 (at most
// 4 + 2 significant bits); the multiply by s_t rounds once, so fp32 output is
// the correctly rounded exact value, and bf16 output is rounded once from
// the exact value using the fma residual.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void k_nv_dequantize(const unsigned* __restrict__ q,
                                                       const uint8_t* __restrict__ s,
                                                       const float* __restrict__ g, void* __restrict__ y,
                                                       int64_t nlanes) {
  // kDeqU chunks of 256 lanes per block, loads first (as k_mx_dequantize)
  const int64_t t0 = (int64_t)blockIdx.x * (256 * kDeqU) + threadIdx.x;
  if (t0 >= nlanes) return;
  const float st = *g;
  unsigned cv[kDeqU], sv[kDeqU];
#pragma unroll
  for (int u = 0; u < kDeqU; u++) {
    const int64_t t = t0 + 256 * u < nlanes ? t0 + 256 * u : t0;
    cv[u] = q[t];
    sv[u] = s[t >> 1];
  }
#pragma unroll
  for (int u = 0; u < kDeqU; u++) {
    const int64_t t = t0 + 256 * u;
    if (t >= nlanes) break;
    const unsigned c = cv[u];
    const float sbv = e4m3_value(sv[u]);
    auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    const float r[8] = {p0[0] * sbv, p0[1] * sbv, p1[0] * sbv, p1[1] * sbv,
                        p2[0] * sbv, p2[1] * sbv, p3[0] * sbv, p3[1] * sbv};
    if (kBf16Out) {
      unsigned short h[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        float p = st * r[i];
        float e = __builtin_fmaf(st, r[i], -p);
        h[i] = bf16_rne_of_sum(p, e);
      }
      u32x4 o = {h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16), h[4] | ((unsigned)h[5] << 16),
                 h[6] | ((unsigned)h[7] << 16)};
      st_stream(&((u32x4*)y)[t], o);
    } else {
      f32x4 o0 = {st * r[0], st * r[1], st * r[2], st * r[3]};
      f32x4 o1 = {st * r[4], st * r[5], st * r[6], st * r[7]};
      st_stream(&((f32x4*)y)[2 * t], o0);
      st_stream(&((f32x4*)y)[2 * t + 1], o1);
    }
  }
}

// ---------------------------------------------------------------- TransFP4 blocks

// TransFP4 [TransFP4 page sec. 2.3 eq. (3): x_hat = H^T Q_f(Hx - P_r Hx) +
// H^T P_r Hx; sec. 3.1: a 32-point Hadamard, at most one residual per 32
// values, and per block the NVFP4 or the INT4 candidate by block error].
// Per 32-block (four lanes):
//   * y = H_32 x as rotate8<32> (the rotated-MXFP4 order);
//   * the residual: the largest |y_i| (first position on ties), stored as
//     bf16 (nearest even) and set to +0 in the block Q_f sees;
//   * two candidates under E4M3 scales per 16 and the fp32 tensor scale
//     s_t = amax' / 2688 of the residual-free rotated tensor, with the
//     NVFP4 order of operations: t = fl(Q s_t), s_b = E4M3(fl(amax_16 / t)),
//     d = fl(s_t s_b), v = fl(y / d) correctly rounded -- the E2M1 codebook
//     with Q = 6, and INT4 (sign and magnitude 0..7, nearest even,
//     saturating) with Q = 7;
//   * block error SSE = sum fl(e^2), e = fl(y - fl(c d)): each lane sums its
//     8 terms in order, then the quad adds (P0 + P1) + (P2 + P3); INT4 is
//     kept only if its SSE is strictly smaller.
// Storage per block: 16 code bytes, two E4M3 scales, a meta byte (bit 7:
// INT4, bits 0-4: residual position) and the bf16 residual.

// Residual of a rotated 32-block: the block position of the largest |v|
// (first on ties) is returned to every lane of the quad; the lane that holds
// it takes the value into rv and zeroes it.
__device__ __forceinline__ int tf4_split(float (&v)[8], int lane, float& rv) {
  const int ql = lane & 3;
  unsigned best = __float_as_uint(v[0]) & 0x7FFFFFFFu;
  unsigned at = 8u * ql;
#pragma unroll
  for (int i = 1; i < 8; i++) {
    const unsigned a = __float_as_uint(v[i]) & 0x7FFFFFFFu;  // |v| orders like its bits
    if (a > best) {
      best = a;
      at = 8u * ql + i;
    }
  }
  {
    const unsigned ob = dpp_quad_xor1(best), oa = dpp_quad_xor1(at);
    const bool take = ob > best || (ob == best && oa < at);
    best = take ? ob : best;
    at = take ? oa : at;
  }
  {
    const unsigned ob = dpp_quad_xor2(best), oa = dpp_quad_xor2(at);
    const bool take = ob > best || (ob == best && oa < at);
    best = take ? ob : best;
    at = take ? oa : at;
  }
  const bool own = (int)(at >> 3) == ql;
  rv = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const bool hit = own && (int)(at & 7u) == i;
    rv = hit ? v[i] : rv;
    v[i] = hit ? 0.0f : v[i];
  }
  return (int)at;
}

__device__ __forceinline__ float quad_xor1_f(float v) { return __uint_as_float(dpp_quad_xor1(__float_as_uint(v))); }
__device__ __forceinline__ float quad_xor2_f(float v) { return __uint_as_float(dpp_quad_xor2(__float_as_uint(v))); }

// One candidate for this lane's 8 residual-free values (16-block amax known):
// packed codes, the E4M3 scale code and the block SSE (same on all 4 lanes).
template <bool kInt4>
__device__ __forceinline__ void tf4_candidate(const float (&v)[8], float amax, float st, unsigned& codes,
                                              unsigned& sb, float& sse) {
  sb = e4m3_encode_nonneg(__fdiv_rn(amax, (kInt4 ? 7.0f : 6.0f) * st));
  const float sbv = e4m3_value(sb);
  float e[8];
  unsigned out = 0;
  if (sbv == 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      out |= (__float_as_uint(v[i]) >> 31) << (3 + 4 * i);
      e[i] = v[i];
    }
  } else {
    const float d = st * sbv;
    float qv[8];
    if (d >= 0x1p-100f && amax <= d * 0x1p100f) {
      const float y = __fdiv_rn(1.0f, d);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const unsigned xb = __float_as_uint(v[i]);
        const float aq = div_by_block_scale(__uint_as_float(xb & 0x7FFFFFFFu), d, y);
        qv[i] = __uint_as_float(__float_as_uint(aq) | (xb & 0x80000000u));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) qv[i] = __fdiv_rn(v[i], d);
    }
    float cv[8];
    if constexpr (kInt4) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float mag = fminf(__builtin_rintf(fabsf(qv[i])), 7.0f);  // nearest, ties to even
        const unsigned sg = __float_as_uint(qv[i]) >> 31;
        out |= (((unsigned)mag) | (sg << 3)) << (4 * i);
        cv[i] = sg ? -mag : mag;
      }
    } else {
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, qv[0], qv[1], 1.0f, 0);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, qv[2], qv[3], 1.0f, 1);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, qv[4], qv[5], 1.0f, 2);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, qv[6], qv[7], 1.0f, 3);
      const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(out, 1.0f, 0);
      const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(out, 1.0f, 1);
      const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(out, 1.0f, 2);
      const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(out, 1.0f, 3);
      cv[0] = p0[0]; cv[1] = p0[1]; cv[2] = p1[0]; cv[3] = p1[1];
      cv[4] = p2[0]; cv[5] = p2[1]; cv[6] = p3[0]; cv[7] = p3[1];
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float dq = cv[i] * d;
      e[i] = v[i] - dq;
    }
  }
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float sq = e[i] * e[i];
    acc = acc + sq;
  }
  acc = acc + quad_xor1_f(acc);  // lanes 0,1: P0 + P1; lanes 2,3: P2 + P3
  acc = acc + quad_xor2_f(acc);  // (P0 + P1) + (P2 + P3) on every lane
  codes = out;
  sse = acc;
}

// Pass 1: per block of this grid, the largest |y'| (residual-free rotated
// values) of its grid-stride share, as fp32 bits, into part[block]; then
// k_nv_scale folds the partials into s_t = amax' / 2688.
// Lane slots per thread per step (loads in flight).  The grid is at most
// kScaleMaxParts = 2048 blocks of 4 waves, 8 waves per SIMD on 256 CUs: it
// fits the chip in one round only if the kernel stays within 64 VGPRs.
// 4 slots took 67 (7 waves per SIMD, so 256 blocks ran as a second round):
// TransFP4 quantize of 16384 x 8192 bf16, interleaved A/B, 238.1 us with 4
// slots, 227.7 with 3 (38 VGPRs), 225.9 with 2 (24 VGPRs); the next step's
// loads issued before the current step's arithmetic measured the same
// (225.4-228.0 us with 1-3 slots).
#ifndef MXQ_TF4A_U
#define MXQ_TF4A_U 2
#endif
constexpr int kTf4U = MXQ_TF4A_U;

template <bool kBf16In>
__global__ __launch_bounds__(256) void k_tf4_amax(const u32x4* __restrict__ x, int64_t nlanes,
                                                  unsigned* __restrict__ part) {
  __shared__ unsigned wmax[4];
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * 256;
  unsigned m = 0;
  // slot u of a step is lane base + u * stride; stride, base - threadIdx.x
  // and nlanes are multiples of 4, so each quad (one 32-block) is whole
  for (int64_t base = (int64_t)blockIdx.x * 256 + threadIdx.x; base - threadIdx.x < nlanes;
       base += kTf4U * stride) {
    float v[kTf4U][8];
#pragma unroll
    for (int u = 0; u < kTf4U; u++) {
      const int64_t t = base + u * stride;
      if (t < nlanes) {
        load8<kBf16In>(x, t, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++) v[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kTf4U; u++) {
      rotate8<32>(v[u], lane);
      // the block's largest |y| once the residual is removed is its second
      // largest |y| counted with multiplicity: a running top two per lane,
      // merged over the quad (|y| orders like its bits)
      unsigned m1 = 0, m2 = 0;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const unsigned a = __float_as_uint(v[u][i]) & 0x7FFFFFFFu;
        m2 = max(m2, min(m1, a));
        m1 = max(m1, a);
      }
      {
        const unsigned p1 = dpp_quad_xor1(m1), p2 = dpp_quad_xor1(m2);
        m2 = max(min(m1, p1), max(m2, p2));
        m1 = max(m1, p1);
      }
      {
        const unsigned p1 = dpp_quad_xor2(m1), p2 = dpp_quad_xor2(m2);
        m2 = max(min(m1, p1), max(m2, p2));
        m1 = max(m1, p1);
      }
      m = max(m, m2);
    }
  }
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

// Pass 2: one lane = 8 elements, a quad = one 32-block, a lane pair = one
// 16-element scale block.
template <bool kBf16In>
__global__ __launch_bounds__(256) void k_tf4_quantize(const u32x4* __restrict__ x, const float* __restrict__ g,
                                                      unsigned* __restrict__ q, uint8_t* __restrict__ s,
                                                      uint8_t* __restrict__ meta, uint16_t* __restrict__ res,
                                                      int64_t nlanes) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nlanes) return;  // nlanes % 4 == 0: quads stay whole
  const int lane = threadIdx.x & 63;
  const float st = *g;
  float v[8];
  load8<kBf16In>(x, t, v);
  rotate8<32>(v, lane);
  float rv;
  const int at = tf4_split(v, lane, rv);
  unsigned m = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  m = max(m, dpp_quad_xor1(m));  // the 16-element half
  const float amax = __uint_as_float(m);
  unsigned cn, ci, sn, si;
  float en, ei;
  tf4_candidate<false>(v, amax, st, cn, sn, en);
  tf4_candidate<true>(v, amax, st, ci, si, ei);
  const bool int4 = ei < en;
  q[t] = int4 ? ci : cn;
  if ((t & 1) == 0) s[t >> 1] = (uint8_t)(int4 ? si : sn);
  if ((t & 3) == 0) meta[t >> 2] = (uint8_t)((int4 ? 0x80u : 0u) | (unsigned)at);
  if ((at >> 3) == (lane & 3)) res[t >> 2] = f32_to_bf16_rne(rv);
}

// Dequantize: y_hat = fl(c * fl(s_t * E4M3(s_b))) with the codebook the tag
// selects, the residual added at its position, then x_hat = H^T y_hat = H
// y_hat (H_32 is symmetric and orthonormal) in the same butterfly order.
// 256-lane chunks per block, loads issued together (16384 x 8192: 128 us
// with one chunk and the residual loaded after the meta byte, 95 us with
// one chunk and every load up front, 74.6 with 2, 70.7 with 4, 80.7 with 8)
#ifndef MXQ_TF4D_U
#define MXQ_TF4D_U 4
#endif
constexpr int kTf4dU = MXQ_TF4D_U;
template <bool kBf16Out>
__global__ __launch_bounds__(256) void k_tf4_dequantize(const unsigned* __restrict__ q,
                                                        const uint8_t* __restrict__ s,
                                                        const uint8_t* __restrict__ meta,
                                                        const uint16_t* __restrict__ res,
                                                        const float* __restrict__ g, void* __restrict__ y,
                                                        int64_t nlanes) {
  const int64_t t0 = (int64_t)blockIdx.x * (256 * kTf4dU) + threadIdx.x;
  if (t0 >= nlanes) return;  // nlanes % 4 == 0 and chunks are 256 lanes: quads stay whole
  const int lane = threadIdx.x & 63;
  // every load of the block's kTf4dU chunks up front, none depending on
  // another (the residual used to be loaded only by the lane holding its
  // position, once the meta byte had arrived: two memory round trips in a
  // row).  Lanes past the end read lane 0's bytes and store nothing.
  const float st = *g;
  unsigned c[kTf4dU], sbyte[kTf4dU], mb[kTf4dU], rbits[kTf4dU];
#pragma unroll
  for (int u = 0; u < kTf4dU; u++) {
    const int64_t t = t0 + 256 * u < nlanes ? t0 + 256 * u : 0;
    c[u] = q[t];
    sbyte[u] = s[t >> 1];
    mb[u] = meta[t >> 2];
    rbits[u] = res[t >> 2];
  }
#pragma unroll
  for (int u = 0; u < kTf4dU; u++) {
    const int64_t t = t0 + 256 * u;
    const float d = st * e4m3_value(sbyte[u]);
    const int at = (int)(mb[u] & 31u);
    float v[8];
    if (mb[u] & 0x80u) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const unsigned ci = (c[u] >> (4 * i)) & 15u;
        const float mag = (float)(ci & 7u);
        v[i] = (ci & 8u) ? -mag : mag;
      }
    } else {
      const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[u], 1.0f, 0);
      const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[u], 1.0f, 1);
      const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[u], 1.0f, 2);
      const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[u], 1.0f, 3);
      v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
      v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
    }
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = v[i] * d;
    {
      const bool own = (at >> 3) == (lane & 3);
      const float rv = __uint_as_float(rbits[u] << 16);
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = own && (at & 7) == i ? v[i] + rv : v[i];
    }
    rotate8<32>(v, lane);
    if (t < nlanes) {
      if (kBf16Out) {
        u32x4 o;
        o.x = f32_to_bf16_rne(v[0]) | ((unsigned)f32_to_bf16_rne(v[1]) << 16);
        o.y = f32_to_bf16_rne(v[2]) | ((unsigned)f32_to_bf16_rne(v[3]) << 16);
        o.z = f32_to_bf16_rne(v[4]) | ((unsigned)f32_to_bf16_rne(v[5]) << 16);
        o.w = f32_to_bf16_rne(v[6]) | ((unsigned)f32_to_bf16_rne(v[7]) << 16);
        st_stream(&((u32x4*)y)[t], o);
      } else {
        st_stream(&((f32x4*)y)[2 * t], (f32x4){v[0], v[1], v[2], v[3]});
        st_stream(&((f32x4*)y)[2 * t + 1], (f32x4){v[4], v[5], v[6], v[7]});
      }
    }
  }
}

// ---------------------------------------------------------------- launchers

static inline unsigned grid_for(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

hipError_t launch_mx_quantize(const void* x, bool bf16, int64_t rows, int64_t k, uint8_t* q, uint8_t* s,
                              hipStream_t st) {
  int64_t nlanes = rows * k / 8;
  if (bf16)
    hipLaunchKernelGGL(k_mx_quantize_bf16, dim3(grid_for(nlanes, 256 * kQuantU)), dim3(256), 0, st,
                       (const u32x4*)x, (unsigned*)q, s, nlanes);
  else
    hipLaunchKernelGGL(k_mx_quantize_f32, dim3(grid_for(nlanes, 256)), dim3(256), 0, st, (const u32x4*)x,
                       (unsigned*)q, s, nlanes);
  return hipGetLastError();
}

hipError_t launch_mx8_quantize(const void* x, bool bf16, int64_t rows, int64_t k, uint8_t* q, uint8_t* s,
                               hipStream_t st) {
  const int64_t nlanes = rows * k / 8;
  if (bf16)
    hipLaunchKernelGGL(k_mx8_quantize_bf16, dim3(grid_for(nlanes, 256 * kQuant8U)), dim3(256), 0, st,
                       (const u32x4*)x, (u32x2*)q, s, nlanes);
  else
    hipLaunchKernelGGL(k_mx8_quantize_f32, dim3(grid_for(nlanes, 256)), dim3(256), 0, st, (const u32x4*)x,
                       (u32x2*)q, s, nlanes);
  return hipGetLastError();
}

template <int HK>
static void launch_mx_quantize_hadamard_hk(const void* x, bool bf16, int64_t nlanes, uint8_t* q, uint8_t* s,
                                           hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL((k_mx_quantize_hadamard<true, HK>), dim3(grid_for(nlanes, 256 * kHadU)), dim3(256), 0, st,
                       (const u32x4*)x, (unsigned*)q, s, nlanes);
  else
    hipLaunchKernelGGL((k_mx_quantize_hadamard<false, HK>), dim3(grid_for(nlanes, 256 * kHadU)), dim3(256), 0, st,
                       (const u32x4*)x, (unsigned*)q, s, nlanes);
}

hipError_t launch_mx_quantize_hadamard(const void* x, bool bf16, int64_t rows, int64_t k, int hk, uint8_t* q,
                                       uint8_t* s, hipStream_t st) {
  const int64_t nlanes = rows * k / 8;
  switch (hk) {
    case 16: launch_mx_quantize_hadamard_hk<16>(x, bf16, nlanes, q, s, st); break;
    case 32: launch_mx_quantize_hadamard_hk<32>(x, bf16, nlanes, q, s, st); break;
    case 64: launch_mx_quantize_hadamard_hk<64>(x, bf16, nlanes, q, s, st); break;
    case 128: launch_mx_quantize_hadamard_hk<128>(x, bf16, nlanes, q, s, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t k, void* y,
                                bool bf16, hipStream_t st) {
  int64_t nlanes = rows * k / 8;
  if (bf16)
    hipLaunchKernelGGL(k_mx_dequantize<true>, dim3(grid_for(nlanes, 256 * kDeqU)), dim3(256), 0, st,
                       (const unsigned*)q, s, y, nlanes);
  else
    hipLaunchKernelGGL(k_mx_dequantize<false>, dim3(grid_for(nlanes, 256 * kDeqU)), dim3(256), 0, st,
                       (const unsigned*)q, s, y, nlanes);
  return hipGetLastError();
}

hipError_t launch_nv_quantize(const void* x, bool bf16, int64_t rows, int64_t k, float* gscale,
                              bool compute_gscale, uint8_t* q, uint8_t* s, hipStream_t st) {
  int64_t n = rows * k;
  int64_t nlanes = n / 8;
  if (compute_gscale) {
    // partials go to the code buffer (rows * k / 2 bytes, at least 8)
    const int64_t nvec = bf16 ? n / 8 : n / 4;
    const int64_t want = (nvec + 256 * kAmaxU - 1) / (256 * kAmaxU);
    const int np = (int)std::max<int64_t>(1, std::min<int64_t>({want, kScaleMaxParts, n / 8}));
    unsigned* part = (unsigned*)q;
    if (bf16)
      hipLaunchKernelGGL(k_nv_amax<true>, dim3(np), dim3(256), 0, st, (const u32x4*)x, nvec, part);
    else
      hipLaunchKernelGGL(k_nv_amax<false>, dim3(np), dim3(256), 0, st, (const u32x4*)x, nvec, part);
    hipLaunchKernelGGL(k_nv_scale, dim3(1), dim3(kScaleThreads), 0, st, (const unsigned*)part, np, gscale);
  }
  if (bf16)
    hipLaunchKernelGGL(k_nv_quantize<true>, dim3(grid_for(nlanes, 256 * kNvqU)), dim3(256), 0, st, (const u32x4*)x,
                       (const float*)gscale, (unsigned*)q, s, nlanes);
  else
    hipLaunchKernelGGL(k_nv_quantize<false>, dim3(grid_for(nlanes, 256 * kNvqU)), dim3(256), 0, st, (const u32x4*)x,
                       (const float*)gscale, (unsigned*)q, s, nlanes);
  return hipGetLastError();
}

hipError_t launch_nv_dequantize(const uint8_t* q, const uint8_t* s, const float* gscale, int64_t rows,
                                int64_t k, void* y, bool bf16, hipStream_t st) {
  int64_t nlanes = rows * k / 8;
  if (bf16)
    hipLaunchKernelGGL(k_nv_dequantize<true>, dim3(grid_for(nlanes, 256 * kDeqU)), dim3(256), 0, st,
                       (const unsigned*)q, s, gscale, y, nlanes);
  else
    hipLaunchKernelGGL(k_nv_dequantize<false>, dim3(grid_for(nlanes, 256 * kDeqU)), dim3(256), 0, st,
                       (const unsigned*)q, s, gscale, y, nlanes);
  return hipGetLastError();
}

hipError_t launch_tf4_quantize(const void* x, bool bf16, int64_t rows, int64_t k, float* gscale,
                               bool compute_gscale, uint8_t* q, uint8_t* s, uint8_t* meta, uint16_t* res,
                               hipStream_t st) {
  const int64_t nlanes = rows * k / 8;
  if (compute_gscale) {
    // partials go to the code buffer (4 * nlanes bytes >= 4 * np)
    const int np = (int)std::max<int64_t>(1, std::min<int64_t>(grid_for(nlanes, 256 * kTf4U), kScaleMaxParts));
    unsigned* part = (unsigned*)q;
    if (bf16)
      hipLaunchKernelGGL(k_tf4_amax<true>, dim3(np), dim3(256), 0, st, (const u32x4*)x, nlanes, part);
    else
      hipLaunchKernelGGL(k_tf4_amax<false>, dim3(np), dim3(256), 0, st, (const u32x4*)x, nlanes, part);
    hipLaunchKernelGGL(k_nv_scale, dim3(1), dim3(kScaleThreads), 0, st, (const unsigned*)part, np, gscale);
  }
  if (bf16)
    hipLaunchKernelGGL(k_tf4_quantize<true>, dim3(grid_for(nlanes, 256)), dim3(256), 0, st, (const u32x4*)x,
                       (const float*)gscale, (unsigned*)q, s, meta, res, nlanes);
  else
    hipLaunchKernelGGL(k_tf4_quantize<false>, dim3(grid_for(nlanes, 256)), dim3(256), 0, st, (const u32x4*)x,
                       (const float*)gscale, (unsigned*)q, s, meta, res, nlanes);
  return hipGetLastError();
}

hipError_t launch_tf4_dequantize(const uint8_t* q, const uint8_t* s, const uint8_t* meta, const uint16_t* res,
                                 const float* gscale, int64_t rows, int64_t k, void* y, bool bf16_out,
                                 hipStream_t st) {
  const int64_t nlanes = rows * k / 8;
  const dim3 grid(grid_for(nlanes, 256 * kTf4dU));
  if (bf16_out)
    hipLaunchKernelGGL(k_tf4_dequantize<true>, grid, dim3(256), 0, st, (const unsigned*)q, s, meta, res, gscale, y,
                       nlanes);
  else
    hipLaunchKernelGGL(k_tf4_dequantize<false>, grid, dim3(256), 0, st, (const unsigned*)q, s, meta, res, gscale, y,
                       nlanes);
  return hipGetLastError();
}

}  // namespace mxq
