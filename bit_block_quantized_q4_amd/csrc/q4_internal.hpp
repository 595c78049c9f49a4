// Internal declarations shared by the libq4 translation units (HIP, gfx950).
// Not installed; the public interface is include/q4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

constexpr int kQK = 32;          // weights per block
constexpr int kBlockBytes = 18;  // fp16 scale + 16 code bytes
constexpr int kWave = 64;        // CDNA wavefront

enum class DType : int { F32 = 0, F16 = 1 };

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

// Launchers (return the launch status; never synchronise).
hipError_t launch_quantize(const void* w, DType wt, int64_t n, int64_t k,
                           uint8_t* packed, hipStream_t s);

hipError_t launch_gemv(const void* x, DType xt, const uint8_t* packed, void* y,
                       DType yt, int m, int64_t n, int64_t k, hipStream_t s);

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();

// Decode GEMV on 16x16x32 matrix cores (k a multiple of 1024, m <= 32).
bool gemv_tile_supports(int m, int64_t k);
hipError_t launch_gemv_tile(const void* x, const uint8_t* packed, void* y, bool y_f16, int m,
                            int64_t n, int64_t k, hipStream_t s);

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm(const void* x, DType xt, const uint8_t* packed, void* y,
                       DType yt, int64_t m, int64_t n, int64_t k,
                       void* workspace, hipStream_t s);

}  // namespace q4
