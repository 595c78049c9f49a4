// Q4_0 batched-decode GEMV for gfx950: y[m][n] = x[m][k] . dequant(W)^T, m <= 32.
//
// The "batch decode" stage of the vertical-disaggregation page (section
// "Every cycle counts: custom kernels"): many sessions' decode steps share one
// pass over the weights, so the kernel reads each packed byte once for all m
// activation rows.  Per block: nibble unpack to exact small integers (q - 8),
// an fp32 dot product with the activations, then one multiply-add by the
// block's scale d into an fp32 accumulator.  A row's partial sums are reduced
// across the wavefront with xor shuffles in a fixed order, so results are
// bit-reproducible.
#include "q4_internal.hpp"

namespace q4 {
namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// One wavefront per output feature n; lane l walks blocks l, l+64, ...
template <typename XT, typename YT, int MT>
__global__ __launch_bounds__(256) void gemv_rowwave_kernel(
    const XT* __restrict__ x, const uint8_t* __restrict__ W, YT* __restrict__ y,
    int m, int64_t n, int64_t k) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) +
                      (threadIdx.x / kWave);
  if (row >= n) return;  // whole wavefront
  const int64_t nb = k / kQK;
  const uint8_t* wr = W + row * nb * kBlockBytes;

  float acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = 0.0f;

  for (int64_t b = lane; b < nb; b += kWave) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(wr + b * kBlockBytes);
    const float d = half_bits_to_float(p[0]);
    float wq[kQK];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = p[1 + i];  // code bytes 2i (low half) and 2i+1
      wq[2 * i] = static_cast<float>(static_cast<int>(c & 0xFu) - 8);
      wq[2 * i + 16] = static_cast<float>(static_cast<int>((c >> 4) & 0xFu) - 8);
      wq[2 * i + 1] = static_cast<float>(static_cast<int>((c >> 8) & 0xFu) - 8);
      wq[2 * i + 17] = static_cast<float>(static_cast<int>((c >> 12) & 0xFu) - 8);
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      if (mi < m) {
        const XT* xr = x + static_cast<int64_t>(mi) * k + b * kQK;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < kQK; ++j) s = fmaf(to_f32(xr[j]), wq[j], s);
        acc[mi] = fmaf(d, s, acc[mi]);
      }
    }
  }

#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) acc[mi] += __shfl_xor(acc[mi], off);
  }
  if (lane == 0) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
      if (mi < m) y[static_cast<int64_t>(mi) * n + row] = from_f32<YT>(acc[mi]);
  }
}

template <typename XT, typename YT, int MT>
hipError_t launch_rowwave(const void* x, const uint8_t* packed, void* y, int m,
                          int64_t n, int64_t k, hipStream_t s) {
  const XT* xp = static_cast<const XT*>(x);
  YT* yp = static_cast<YT*>(y);
  void* argv[] = {&xp, const_cast<const uint8_t**>(&packed), &yp, &m, &n, &k};
  const dim3 grid(static_cast<unsigned>((n + 3) / 4));
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_rowwave_kernel<XT, YT, MT>),
                         grid, dim3(256), argv, 0, s);
}

template <typename XT, typename YT>
hipError_t dispatch_m(const void* x, const uint8_t* packed, void* y, int m,
                      int64_t n, int64_t k, hipStream_t s) {
  if (m <= 1) return launch_rowwave<XT, YT, 1>(x, packed, y, m, n, k, s);
  if (m <= 2) return launch_rowwave<XT, YT, 2>(x, packed, y, m, n, k, s);
  if (m <= 4) return launch_rowwave<XT, YT, 4>(x, packed, y, m, n, k, s);
  if (m <= 8) return launch_rowwave<XT, YT, 8>(x, packed, y, m, n, k, s);
  if (m <= 16) return launch_rowwave<XT, YT, 16>(x, packed, y, m, n, k, s);
  return launch_rowwave<XT, YT, 32>(x, packed, y, m, n, k, s);
}

}  // namespace

hipError_t launch_gemv(const void* x, DType xt, const uint8_t* packed, void* y,
                       DType yt, int m, int64_t n, int64_t k, hipStream_t s) {
  if (xt == DType::F16) {
    if (yt == DType::F16) return dispatch_m<half_t, half_t>(x, packed, y, m, n, k, s);
    return dispatch_m<half_t, float>(x, packed, y, m, n, k, s);
  }
  if (yt == DType::F16) return dispatch_m<float, half_t>(x, packed, y, m, n, k, s);
  return dispatch_m<float, float>(x, packed, y, m, n, k, s);
}

}  // namespace q4
