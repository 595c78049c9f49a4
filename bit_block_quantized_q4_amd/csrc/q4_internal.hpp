// Internal declarations shared by the libq4 translation units (HIP, gfx950).
// Not installed; the public interface is include/q4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace q4 {

constexpr int kQK = 32;          // weights per block
constexpr int kBlockBytes = 18;  // fp16 scale + 16 code bytes
constexpr int kWave = 64;        // CDNA wavefront

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// fp16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float half_bits_to_float(uint16_t bits) {
  return static_cast<float>(__builtin_bit_cast(half_t, bits));
}

// bfloat16 storage: the upper half of an IEEE binary32 pattern.
struct bf16_t {
  uint16_t bits;
};

// bf16 bit pattern -> fp32 (exact: the pattern shifted into the upper half).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits) {
  return __builtin_bit_cast(float, bits << 16);
}

// Two bf16 values packed in a dword (element 0 in the low half) -> the same
// two values as fp16, rounded to nearest even: exact for every value fp16
// represents (all bf16 values with 2^-14 <= |v| <= 65504 among them).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  const float lo = __builtin_bit_cast(float, v << 16);
  const float hi = __builtin_bit_cast(float, v & 0xFFFF0000u);
  const half2_t h = {static_cast<half_t>(lo), static_cast<half_t>(hi)};
  return __builtin_bit_cast(uint32_t, h);
}

// Whether the fp16 pair h (from bf16x2_to_f16x2) denotes exactly the bf16
// pair v: false where fp16 overflowed or rounded (out of fp16's range or off
// its subnormal grid) and for NaN.
__device__ __forceinline__ bool f16x2_holds_bf16x2(uint32_t h, uint32_t v) {
  const half2_t hh = __builtin_bit_cast(half2_t, h);
  return static_cast<float>(hh[0]) == __builtin_bit_cast(float, v << 16) &&
         static_cast<float>(hh[1]) == __builtin_bit_cast(float, v & 0xFFFF0000u);
}

// Allows kernel `fn` up to `bytes` of dynamic LDS on the current device, once
// per device (bit d of `done` records device d; devices past 63 set it on
// every launch).  Safe to call from several host threads at once.
inline hipError_t allow_dynamic_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return ge;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Launchers (return the launch status; never synchronise).
hipError_t launch_quantize(const void* w, DType wt, int64_t n, int64_t k,
                           uint8_t* packed, hipStream_t s);

hipError_t launch_gemv(const void* x, DType xt, const uint8_t* packed, void* y,
                       DType yt, int m, int64_t n, int64_t k, hipStream_t s);

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();

// Decode GEMV on 16x16x32 matrix cores (k a multiple of 512, m <= 32).
bool gemv_tile_supports(int m, int64_t k);
hipError_t launch_gemv_tile(const void* x, bool x_bf16, const uint8_t* packed, void* y,
                            bool y_f16, int m, int64_t n, int64_t k, hipStream_t s);

// Workspace of a GEMM whose activations have dtype xt: bf16 activations are
// first converted to fp16 into its leading m * k * 2 bytes (rounded up to 256).
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, DType xt);
hipError_t launch_gemm(const void* x, DType xt, const uint8_t* packed, void* y,
                       DType yt, int64_t m, int64_t n, int64_t k,
                       void* workspace, hipStream_t s);

}  // namespace q4
