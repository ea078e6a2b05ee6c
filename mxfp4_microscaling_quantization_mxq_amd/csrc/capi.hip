// capi.hip -- the library's C ABI (declared in include/mxq.h): argument
// validation, device check, and kernel launch.  Every check runs on the host
// before anything is enqueued; on an error nothing is written.
#include <string.h>

#include <atomic>

#include "../../include/mxq.h"
#include "mxq_launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch_ok[kMaxDevices];

mxq_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return MXQ_ERROR_NOT_SUPPORTED;
  }
  if (dev >= kMaxDevices) return MXQ_ERROR_NOT_SUPPORTED;
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return MXQ_ERROR_NOT_SUPPORTED;
    }
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? MXQ_SUCCESS : MXQ_ERROR_NOT_SUPPORTED;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

mxq_status launched(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MXQ_ERROR_LAUNCH_FAILURE;
  }
  return MXQ_SUCCESS;
}

bool valid_dtype(mxq_dtype d) { return d == MXQ_F32 || d == MXQ_BF16; }

// Grid limits of the launchers (1-D grids of 256-thread blocks over 8-element
// lanes; the product kernels put m in grid.y).
constexpr int64_t kMaxElems = (int64_t)0x7FFFFFFF * 256 * 8;
constexpr int64_t kMaxGridY = 65535;

}  // namespace

extern "C" {

const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_SUCCESS: return "success";
    case MXQ_ERROR_INVALID_VALUE: return "invalid value (null pointer, a size below 1, or k not a multiple of the block size)";
    case MXQ_ERROR_MISALIGNED: return "misaligned pointer (16-byte alignment required)";
    case MXQ_ERROR_NOT_SUPPORTED: return "not supported (no HIP device, or the device is not gfx950)";
    case MXQ_ERROR_LAUNCH_FAILURE: return "kernel launch failed";
    default: break;
  }
  return "unknown status";
}

int mxq_version(void) { return 200; }

// Every size must be at least 1: an empty problem is an invalid argument,
// not a no-op, so a caller's shape bug surfaces at the call.

mxq_status mxq_quantize(const void* x, mxq_dtype xdt, int64_t rows, int64_t k, uint8_t* q, uint8_t* s,
                        hipStream_t stream) {
  if (rows < 1 || k < 1 || k % 32 != 0 || !valid_dtype(xdt)) return MXQ_ERROR_INVALID_VALUE;
  if (rows > kMaxElems / k) return MXQ_ERROR_INVALID_VALUE;
  if (!x || !q || !s) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_mx_quantize(x, xdt == MXQ_BF16, rows, k, q, s, stream));
}

mxq_status mxq_quantize_hadamard(const void* x, mxq_dtype xdt, int64_t rows, int64_t k, int hk, uint8_t* q,
                                 uint8_t* s, hipStream_t stream) {
  if (hk != 16 && hk != 32 && hk != 64 && hk != 128) return MXQ_ERROR_INVALID_VALUE;
  if (rows < 1 || k < 1 || k % 32 != 0 || k % hk != 0 || !valid_dtype(xdt)) return MXQ_ERROR_INVALID_VALUE;
  if (rows > kMaxElems / k) return MXQ_ERROR_INVALID_VALUE;
  if (!x || !q || !s) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_mx_quantize_hadamard(x, xdt == MXQ_BF16, rows, k, hk, q, s, stream));
}

mxq_status mxq_quantize_fp8(const void* x, mxq_dtype xdt, int64_t rows, int64_t k, uint8_t* q, uint8_t* s,
                            hipStream_t stream) {
  if (rows < 1 || k < 1 || k % 32 != 0 || !valid_dtype(xdt)) return MXQ_ERROR_INVALID_VALUE;
  if (rows > kMaxElems / k) return MXQ_ERROR_INVALID_VALUE;
  if (!x || !q || !s) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_mx8_quantize(x, xdt == MXQ_BF16, rows, k, q, s, stream));
}

mxq_status mxq_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t k, void* y, mxq_dtype ydt,
                          hipStream_t stream) {
  if (rows < 1 || k < 1 || k % 32 != 0 || !valid_dtype(ydt)) return MXQ_ERROR_INVALID_VALUE;
  if (rows > kMaxElems / k) return MXQ_ERROR_INVALID_VALUE;
  if (!q || !s || !y) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(s) || !aligned16(y)) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_mx_dequantize(q, s, rows, k, y, ydt == MXQ_BF16, stream));
}

static mxq_status w4a16_common(bool nv, const uint8_t* wq, const uint8_t* ws, const float* gs, int64_t n,
                               int64_t k, const void* x, int64_t m, void* y, mxq_dtype ydt, hipStream_t stream) {
  const int64_t blk = nv ? 16 : 32;
  if (n < 1 || k < 1 || m < 1 || k % blk != 0 || !valid_dtype(ydt)) return MXQ_ERROR_INVALID_VALUE;
  if ((m + 15) / 16 > kMaxGridY || n > kMaxElems / 16) return MXQ_ERROR_INVALID_VALUE;
  if (!wq || !ws || !x || !y || (nv && !gs)) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(wq) || !aligned16(ws) || !aligned16(x) || !aligned16(y)) return MXQ_ERROR_MISALIGNED;
  if (nv && ((uintptr_t)gs & 3u)) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_w4a16(nv, wq, ws, gs, n, k, x, m, y, ydt == MXQ_BF16, stream));
}

mxq_status mxq_gemv_w4a16(const uint8_t* wq, const uint8_t* ws, int64_t n, int64_t k, const void* x, int64_t m,
                          void* y, mxq_dtype ydt, hipStream_t stream) {
  return w4a16_common(false, wq, ws, nullptr, n, k, x, m, y, ydt, stream);
}

mxq_status nvq_gemm(const uint8_t* wq, const uint8_t* ws, const float* wgscale, int64_t n, int64_t k,
                    const void* x, int64_t m, void* y, mxq_dtype ydt, hipStream_t stream) {
  return w4a16_common(true, wq, ws, wgscale, n, k, x, m, y, ydt, stream);
}

// Shared checks of the block-scaled products (A codes of either format).
static mxq_status product_args(const void* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                               int64_t n, int64_t k, const void* c) {
  if (m < 1 || n < 1 || k < 1 || k % 32 != 0) return MXQ_ERROR_INVALID_VALUE;
  if ((m + 127) / 128 > kMaxGridY || n > kMaxElems / 16) return MXQ_ERROR_INVALID_VALUE;
  if (!aq || !as || !bq || !bs || !c) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(aq) || !aligned16(as) || !aligned16(bq) || !aligned16(bs) || !aligned16(c))
    return MXQ_ERROR_MISALIGNED;
  return MXQ_SUCCESS;
}

mxq_status mxq_gemm_w4a4(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                         int64_t n, int64_t k, void* c, mxq_dtype cdt, hipStream_t stream) {
  if (!valid_dtype(cdt)) return MXQ_ERROR_INVALID_VALUE;
  mxq_status e = product_args(aq, as, bq, bs, m, n, k, c);
  if (e == MXQ_SUCCESS) e = check_device();
  if (e != MXQ_SUCCESS) return e;
  return launched(mxq::launch_w4a4(aq, as, bq, bs, m, n, k, c, cdt == MXQ_BF16, stream));
}

mxq_status mxq_gemm_w4a8(const uint8_t* aq8, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                         int64_t n, int64_t k, void* c, mxq_dtype cdt, hipStream_t stream) {
  if (!valid_dtype(cdt)) return MXQ_ERROR_INVALID_VALUE;
  mxq_status e = product_args(aq8, as, bq, bs, m, n, k, c);
  if (e == MXQ_SUCCESS) e = check_device();
  if (e != MXQ_SUCCESS) return e;
  return launched(mxq::launch_w4a8(aq8, as, bq, bs, m, n, k, c, cdt == MXQ_BF16, stream));
}

mxq_status mxq_gemm_w4a4_quant(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, int64_t m,
                               int64_t n, int64_t k, uint8_t* cq, uint8_t* cs, hipStream_t stream) {
  mxq_status e = product_args(aq, as, bq, bs, m, n, k, cq);
  if (e != MXQ_SUCCESS) return e;
  if (n % 32 != 0 || !cs) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(cs)) return MXQ_ERROR_MISALIGNED;
  e = check_device();
  if (e != MXQ_SUCCESS) return e;
  return launched(mxq::launch_w4a4_mx(aq, as, bq, bs, m, n, k, cq, cs, stream));
}

// The in-GEMM activation quantize serves decode-sized batches only.
static mxq_status dynamic_args(const void* x, const uint8_t* bq, const uint8_t* bs, int64_t m, int64_t n, int64_t k,
                               const void* c, mxq_dtype cdt) {
  if (m < 1 || n < 1 || k < 1 || !valid_dtype(cdt)) return MXQ_ERROR_INVALID_VALUE;
  if (m > 16 || k % 512 != 0 || k > (1 << 24) || n > kMaxElems / 16) return MXQ_ERROR_INVALID_VALUE;
  if (!x || !bq || !bs || !c) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(bq) || !aligned16(bs) || !aligned16(c)) return MXQ_ERROR_MISALIGNED;
  return MXQ_SUCCESS;
}

mxq_status mxq_gemm_w4a4_dynamic(const void* x, const uint8_t* bq, const uint8_t* bs, int64_t m, int64_t n,
                                 int64_t k, void* c, mxq_dtype cdt, hipStream_t stream) {
  mxq_status e = dynamic_args(x, bq, bs, m, n, k, c, cdt);
  if (e == MXQ_SUCCESS) e = check_device();
  if (e != MXQ_SUCCESS) return e;
  return launched(mxq::launch_w4a4_dynamic((const uint16_t*)x, bq, bs, m, n, k, c, cdt == MXQ_BF16, stream));
}

mxq_status mxq_gemm_w4a8_dynamic(const void* x, const uint8_t* bq, const uint8_t* bs, int64_t m, int64_t n,
                                 int64_t k, void* c, mxq_dtype cdt, hipStream_t stream) {
  mxq_status e = dynamic_args(x, bq, bs, m, n, k, c, cdt);
  if (e == MXQ_SUCCESS) e = check_device();
  if (e != MXQ_SUCCESS) return e;
  return launched(mxq::launch_w4a8_dynamic((const uint16_t*)x, bq, bs, m, n, k, c, cdt == MXQ_BF16, stream));
}

mxq_status nvq_quantize(const void* x, mxq_dtype xdt, int64_t rows, int64_t k, float* gscale, int compute_gscale,
                        uint8_t* q, uint8_t* s, hipStream_t stream) {
  if (rows < 1 || k < 1 || k % 16 != 0 || !valid_dtype(xdt)) return MXQ_ERROR_INVALID_VALUE;
  if (rows > kMaxElems / k) return MXQ_ERROR_INVALID_VALUE;
  if (!x || !q || !s || !gscale) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return MXQ_ERROR_MISALIGNED;
  if ((uintptr_t)gscale & 3u) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_nv_quantize(x, xdt == MXQ_BF16, rows, k, gscale, compute_gscale != 0, q, s, stream));
}

mxq_status nvq_dequantize(const uint8_t* q, const uint8_t* s, const float* gscale, int64_t rows, int64_t k, void* y,
                          mxq_dtype ydt, hipStream_t stream) {
  if (rows < 1 || k < 1 || k % 16 != 0 || !valid_dtype(ydt)) return MXQ_ERROR_INVALID_VALUE;
  if (rows > kMaxElems / k) return MXQ_ERROR_INVALID_VALUE;
  if (!q || !s || !gscale || !y) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(s) || !aligned16(y)) return MXQ_ERROR_MISALIGNED;
  if ((uintptr_t)gscale & 3u) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_nv_dequantize(q, s, gscale, rows, k, y, ydt == MXQ_BF16, stream));
}

mxq_status mxq_transfp4_quantize(const void* x, mxq_dtype xdt, int64_t rows, int64_t k, float* gscale,
                                 int compute_gscale, uint8_t* q, uint8_t* s, uint8_t* meta, uint16_t* res,
                                 hipStream_t stream) {
  if (rows < 1 || k < 1 || k % 32 != 0 || !valid_dtype(xdt)) return MXQ_ERROR_INVALID_VALUE;
  if (rows > kMaxElems / k) return MXQ_ERROR_INVALID_VALUE;
  if (!x || !q || !s || !meta || !res || !gscale) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s) || !aligned16(meta) || !aligned16(res))
    return MXQ_ERROR_MISALIGNED;
  if ((uintptr_t)gscale & 3u) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_tf4_quantize(x, xdt == MXQ_BF16, rows, k, gscale, compute_gscale != 0, q, s, meta,
                                           res, stream));
}

mxq_status mxq_transfp4_dequantize(const uint8_t* q, const uint8_t* s, const uint8_t* meta, const uint16_t* res,
                                   const float* gscale, int64_t rows, int64_t k, void* y, mxq_dtype ydt,
                                   hipStream_t stream) {
  if (rows < 1 || k < 1 || k % 32 != 0 || !valid_dtype(ydt)) return MXQ_ERROR_INVALID_VALUE;
  if (rows > kMaxElems / k) return MXQ_ERROR_INVALID_VALUE;
  if (!q || !s || !meta || !res || !gscale || !y) return MXQ_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(s) || !aligned16(meta) || !aligned16(res) || !aligned16(y))
    return MXQ_ERROR_MISALIGNED;
  if ((uintptr_t)gscale & 3u) return MXQ_ERROR_MISALIGNED;
  mxq_status d = check_device();
  if (d != MXQ_SUCCESS) return d;
  return launched(mxq::launch_tf4_dequantize(q, s, meta, res, gscale, rows, k, y, ydt == MXQ_BF16, stream));
}

}  // extern "C"
