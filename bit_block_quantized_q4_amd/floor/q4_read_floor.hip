// A plain streaming read of device memory (include/q4_read_floor.h): 16-byte
// loads, grid-stride, four independent loads in flight per thread, each
// thread's XOR of its data stored once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_read_floor.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_floor_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= p[i];
  sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" int q4_read_floor(const void* p, size_t bytes, uint32_t* sink, int workgroups,
                             void* stream) {
  if (!p || !sink || workgroups < 1) return 1;
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0 || (bytes & 15u) != 0) return 1;
  const u32x4* src = static_cast<const u32x4*>(p);
  int64_t n16 = static_cast<int64_t>(bytes / 16);
  void* argv[] = {&src, &n16, &sink};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&read_floor_kernel),
                                       dim3(static_cast<unsigned>(workgroups)), dim3(256), argv, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : 5;
}
