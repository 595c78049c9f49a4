// The matrix cores' sustained rate (include/q4_mfma_ceiling.h): 8 waves per
// workgroup, each step four A and two B fragments read from LDS per 8
// v_mfma_f32_32x32x16_f16, the reads for step s + 1 interleaved with the
// products of step s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_mfma_ceiling.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kHalves = 32768;   // 64 KB of LDS
constexpr int kWindow = 4096;    // halves read per step
constexpr int kThreads = 512;

__device__ __forceinline__ uint16_t value_bits(uint32_t i, uint32_t seed) {
  uint32_t z = i * 0x9E3779B1u ^ seed;
  z ^= z >> 15;
  z *= 0x2C1B3C6Du;
  z ^= z >> 12;
  z *= 0x297A2D39u;
  z ^= z >> 15;
  return static_cast<uint16_t>((z & 0x8000u) | ((14u + ((z >> 10) & 1u)) << 10) | (z & 0x3FFu));
}

__global__ __launch_bounds__(kThreads, 1) void mfma_ceiling_kernel(uint32_t seed, int iters,
                                                                    float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kHalves];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < kHalves; i += kThreads) lds[i] = value_bits(static_cast<uint32_t>(i), seed);
  __syncthreads();

  // Fragment reads of step s: window 4096 (s % 8), A_i at 512 i + 8 lane,
  // B_j at 2048 + 512 j + 8 lane (at most 7 * 4096 + 3072 + 512 halves).
  const uint16_t* const base = lds + 8 * lane;
  auto read = [&](int s, half8_t (&a)[4], half8_t (&b)[2]) {
    const uint16_t* w = base + (s & 7) * kWindow;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const half8_t*>(w + 512 * i);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const half8_t*>(w + 2048 + 512 * j);
  };
  float16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  half8_t a[4], b[2];
  read(0, a, b);
  for (int s = 0; s < iters; ++s) {
    half8_t na[4], nb[2];
    read(s + 1, na, nb);  // the last step's reads are of valid LDS and unused
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    // each product followed by one fragment read
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = na[i];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = nb[j];
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  sink[static_cast<int64_t>(blockIdx.x) * kThreads + tid] = sum;
}

}  // namespace

extern "C" int q4_mfma_ceiling(uint32_t seed, int iters, float* sink, int workgroups,
                               void* stream) {
  if (!sink || workgroups < 1 || iters < 1) return 1;
  void* argv[] = {&seed, &iters, &sink};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mfma_ceiling_kernel),
                                       dim3(static_cast<unsigned>(workgroups)), dim3(kThreads),
                                       argv, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : 5;
}
