// libq4 C ABI: argument validation and dispatch.  Every check runs on the host
// before anything touches the device; the library keeps no state, never
// allocates, frees or synchronises.
#include <mutex>

#include "q4.h"
#include "q4_internal.hpp"

// Workspace of q4_gemm_noalloc: one copy per device that loads the library,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address is looked up per
// device with hipGetSymbolAddress and only that address reaches a kernel.
static __device__ __align__(256) uint8_t scratch[Q4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxRows = int64_t(1) << 31;
// Largest k of a matmul: the kernels address a tile's rows of x and of the
// packed weight with 32-bit per-lane byte offsets (up to 128 rows of 2 k
// bytes of activations), which stay below 2^32 for k <= 2^24.
constexpr int64_t kMaxMatmulK = int64_t(1) << 24;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Inputs (weights, activations) may be bf16; outputs are fp32 or fp16.
bool valid_in_dtype(int dt) { return dt == Q4_F32 || dt == Q4_F16 || dt == Q4_BF16; }
bool valid_out_dtype(int dt) { return dt == Q4_F32 || dt == Q4_F16; }

size_t dtype_bytes(int dt) { return dt == Q4_F32 ? 4 : 2; }

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a);
  const uintptr_t pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

bool valid_nk(int64_t n, int64_t k) {
  return n >= 1 && k >= Q4_QK && k % Q4_QK == 0 && n < kMaxRows &&
         k < kMaxElems && n <= kMaxElems / k;
}

q4_status from_hip(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per
// device (each device holds its own copy at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

q4_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return Q4_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return Q4_OK;
}

q4_status check_matmul(const void* x, int x_dtype, const void* packed, void* y,
                       int y_dtype, int64_t m, int64_t n, int64_t k) {
  if (!x || !packed || !y) return Q4_ERR_INVALID_ARG;
  if (!valid_nk(n, k) || k > kMaxMatmulK || m < 1 || m >= kMaxRows || m > kMaxElems / k ||
      m > kMaxElems / n)
    return Q4_ERR_SHAPE;
  if (!valid_in_dtype(x_dtype) || !valid_out_dtype(y_dtype)) return Q4_ERR_DTYPE;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(y)) return Q4_ERR_ALIGNMENT;
  const size_t ybytes = static_cast<size_t>(m) * n * dtype_bytes(y_dtype);
  const size_t xbytes = static_cast<size_t>(m) * k * dtype_bytes(x_dtype);
  if (overlap(y, ybytes, x, xbytes) || overlap(y, ybytes, packed, q4_packed_size(n, k)))
    return Q4_ERR_INVALID_ARG;
  return Q4_OK;
}

}  // namespace

extern "C" {

int q4_abi_version(void) { return Q4_ABI_VERSION; }

const char* q4_status_string(int status) {
  switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_INVALID_ARG: return "invalid argument (null pointer or overlapping buffers)";
    case Q4_ERR_SHAPE: return "invalid shape (need m, n >= 1, k >= 32, k % 32 == 0, within size limits)";
    case Q4_ERR_DTYPE: return "unsupported dtype for this call";
    case Q4_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case Q4_ERR_HIP: return "HIP runtime refused the kernel launch";
    case Q4_ERR_WORKSPACE: return "workspace missing or too small";
    case Q4_ERR_UNSUPPORTED: return "the host CPU lacks AVX2, FMA or F16C";
    case Q4_ERR_SCRATCH: return "the call needs more scratch than q4_gemm_noalloc's fixed array holds";
    default: return "unknown q4 status";
  }
}

size_t q4_packed_size(int64_t n, int64_t k) {
  if (!valid_nk(n, k)) return 0;
  return static_cast<size_t>(n) * static_cast<size_t>(k / Q4_QK) * Q4_BLOCK_BYTES;
}

q4_status q4_quantize(const void* w, int w_dtype, int64_t n, int64_t k, void* packed,
                      q4_stream_t stream) {
  if (!w || !packed) return Q4_ERR_INVALID_ARG;
  if (!valid_nk(n, k)) return Q4_ERR_SHAPE;
  if (!valid_in_dtype(w_dtype)) return Q4_ERR_DTYPE;
  if (!aligned16(w) || !aligned16(packed)) return Q4_ERR_ALIGNMENT;
  if (overlap(w, static_cast<size_t>(n) * k * dtype_bytes(w_dtype), packed,
              q4_packed_size(n, k)))
    return Q4_ERR_INVALID_ARG;
  return from_hip(q4::launch_quantize(w, static_cast<q4::DType>(w_dtype), n, k,
                                      static_cast<uint8_t*>(packed),
                                      reinterpret_cast<hipStream_t>(stream)));
}

q4_status q4_gemv(const void* x, int x_dtype, const void* packed, void* y, int y_dtype,
                  int64_t m, int64_t n, int64_t k, q4_stream_t stream) {
  const q4_status st = check_matmul(x, x_dtype, packed, y, y_dtype, m, n, k);
  if (st != Q4_OK) return st;
  if (m > Q4_GEMV_MAX_M) return Q4_ERR_SHAPE;
  return from_hip(q4::launch_gemv(x, static_cast<q4::DType>(x_dtype),
                                  static_cast<const uint8_t*>(packed), y,
                                  static_cast<q4::DType>(y_dtype), static_cast<int>(m),
                                  n, k, reinterpret_cast<hipStream_t>(stream)));
}

size_t q4_gemm_workspace_size(int64_t m, int64_t n, int64_t k) {
  return q4_gemm_workspace_size_dt(m, n, k, Q4_F16);
}

size_t q4_gemm_workspace_size_dt(int64_t m, int64_t n, int64_t k, int x_dtype) {
  if (!valid_nk(n, k) || k > kMaxMatmulK || m < 1 || m >= kMaxRows || m > kMaxElems / k)
    return 0;
  if (!valid_in_dtype(x_dtype)) return 0;
  return q4::gemm_workspace_bytes(m, n, k, static_cast<q4::DType>(x_dtype));
}

q4_status q4_gemm(const void* x, int x_dtype, const void* packed, void* y, int y_dtype,
                  int64_t m, int64_t n, int64_t k, void* workspace,
                  size_t workspace_bytes, q4_stream_t stream) {
  const q4_status st = check_matmul(x, x_dtype, packed, y, y_dtype, m, n, k);
  if (st != Q4_OK) return st;
  const size_t need = q4::gemm_workspace_bytes(m, n, k, static_cast<q4::DType>(x_dtype));
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return Q4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return Q4_ERR_ALIGNMENT;
    const size_t xbytes = static_cast<size_t>(m) * k * dtype_bytes(x_dtype);
    if (overlap(workspace, need, x, xbytes) || overlap(workspace, need, y,
                static_cast<size_t>(m) * n * dtype_bytes(y_dtype)) ||
        overlap(workspace, need, packed, q4_packed_size(n, k)))
      return Q4_ERR_INVALID_ARG;
  }
  return from_hip(q4::launch_gemm(x, static_cast<q4::DType>(x_dtype),
                                  static_cast<const uint8_t*>(packed),
                                  y, static_cast<q4::DType>(y_dtype), m, n, k,
                                  need > 0 ? workspace : nullptr,
                                  reinterpret_cast<hipStream_t>(stream)));
}

q4_status q4_gemm_noalloc(const void* x, int x_dtype, const void* packed, void* y,
                          int y_dtype, int64_t m, int64_t n, int64_t k, q4_stream_t stream) {
  const q4_status st = check_matmul(x, x_dtype, packed, y, y_dtype, m, n, k);
  if (st != Q4_OK) return st;
  const size_t need = q4::gemm_workspace_bytes(m, n, k, static_cast<q4::DType>(x_dtype));
  if (need > Q4_NOALLOC_SCRATCH_BYTES) return Q4_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const q4_status sa = scratch_address(&ws);
    if (sa != Q4_OK) return sa;
  }
  return from_hip(q4::launch_gemm(x, static_cast<q4::DType>(x_dtype),
                                  static_cast<const uint8_t*>(packed),
                                  y, static_cast<q4::DType>(y_dtype), m, n, k, ws,
                                  reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
