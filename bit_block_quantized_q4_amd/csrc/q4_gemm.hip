// Q4_0 prefill GEMM for gfx950: y[m][n] = x[m][k] . dequant(W)^T on fp16 MFMA.
//
// The "GPU Q4_0 -> Tensor Core path" of the vertical-disaggregation page
// (section "Every cycle counts: custom kernels"): long prompts are dense
// computation, so the weight tiles are dequantised once per workgroup into
// LDS as fp16 w = (q - 8) * d (one rounding) and contracted with the fp16
// activations on v_mfma_f32_32x32x16_f16 with fp32 accumulation.  Each output
// element is owned by exactly one lane and accumulated in a fixed k order, so
// results are bit-reproducible.
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int BM = 128;       // rows of x per workgroup
constexpr int BN = 128;       // output features per workgroup
constexpr int BK = kQK;       // one Q4_0 block per k step
constexpr int LDK = BK + 8;   // padded LDS row (halves)

template <typename YT>
__global__ __launch_bounds__(256) void gemm_tile_kernel(
    const half_t* __restrict__ x, const uint8_t* __restrict__ W, YT* __restrict__ y,
    int64_t m, int64_t n, int64_t k) {
  __shared__ __attribute__((aligned(16))) half_t As[BM][LDK];
  __shared__ __attribute__((aligned(16))) half_t Bs[BN][LDK];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wid = t >> 6;
  const int wm = wid >> 1;  // 2 x 2 waves, 64 x 64 each
  const int wn = wid & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t nb = k / kQK;

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int lr = t >> 1;          // tile row this thread stages
  const int lh = t & 1;           // which half of the 32-wide k step

  for (int64_t kb = 0; kb < nb; ++kb) {
    // Activations: 16 halves per thread.
    {
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
      const int64_t gr = m0 + lr;
      if (gr < m) {
        const uint4* src = reinterpret_cast<const uint4*>(x + gr * k + kb * kQK + lh * 16);
        v0 = src[0];
        v1 = src[1];
      }
      *reinterpret_cast<uint4*>(&As[lr][lh * 16]) = v0;
      *reinterpret_cast<uint4*>(&As[lr][lh * 16 + 8]) = v1;
    }
    // Weights: half a block per thread, dequantised to fp16.
    {
      half_t lo[8], hi[8];
      const int64_t gn = n0 + lr;
      if (gn < n) {
        const uint16_t* p =
            reinterpret_cast<const uint16_t*>(W + (gn * nb + kb) * kBlockBytes);
        const float d = half_bits_to_float(p[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t c = p[1 + 4 * lh + i];  // code bytes 8lh+2i, 8lh+2i+1
          lo[2 * i] = static_cast<half_t>(static_cast<float>(static_cast<int>(c & 0xFu) - 8) * d);
          lo[2 * i + 1] = static_cast<half_t>(static_cast<float>(static_cast<int>((c >> 8) & 0xFu) - 8) * d);
          hi[2 * i] = static_cast<half_t>(static_cast<float>(static_cast<int>((c >> 4) & 0xFu) - 8) * d);
          hi[2 * i + 1] = static_cast<half_t>(static_cast<float>(static_cast<int>((c >> 12) & 0xFu) - 8) * d);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) { lo[i] = 0; hi[i] = 0; }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Bs[lr][8 * lh + i] = lo[i];
        Bs[lr][16 + 8 * lh + i] = hi[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      half8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const half8_t*>(&As[wm * 64 + i * 32 + (lane & 31)][ks + 8 * (lane >> 5)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const half8_t*>(&Bs[wn * 64 + j * 32 + (lane & 31)][ks + 8 * (lane >> 5)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: lane l holds column l % 32; register r holds
  // row 8 * (r / 4) + 4 * (l / 32) + r % 4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < m && col < n) y[row * n + col] = static_cast<YT>(acc[i][j][r]);
      }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm(const void* x, DType, const uint8_t* packed, void* y,
                       DType yt, int64_t m, int64_t n, int64_t k, void*,
                       hipStream_t s) {
  const half_t* xp = static_cast<const half_t*>(x);
  const dim3 grid(static_cast<unsigned>((n + BN - 1) / BN),
                  static_cast<unsigned>((m + BM - 1) / BM));
  if (yt == DType::F16) {
    half_t* yp = static_cast<half_t*>(y);
    void* argv[] = {&xp, const_cast<const uint8_t**>(&packed), &yp, &m, &n, &k};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_tile_kernel<half_t>),
                           grid, dim3(256), argv, 0, s);
  }
  float* yp = static_cast<float*>(y);
  void* argv[] = {&xp, const_cast<const uint8_t**>(&packed), &yp, &m, &n, &k};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_tile_kernel<float>),
                         grid, dim3(256), argv, 0, s);
}

}  // namespace q4
