// Q4_0 quantiser for gfx950.
//
// One weight copy serves every backend (vertical-disaggregation page, section
// "Every cycle counts: custom kernels"), so this kernel must reproduce the
// format rule bit for bit: per 32-wide block along K, m is the element of
// largest magnitude (first index on a tie), d = fp16(m / -8) rounded to
// nearest even with subnormals kept, q = min(15, trunc(x / d + 8.5)) with a
// correctly rounded fp32 division by d widened to fp32 and an fp32 add; every
// q is 8 when d is zero.  Bytes: d little-endian, then byte i = q[i] | q[i+16]<<4.
//
// Mapping: eight lanes per block, lane p holds elements 4p..4p+3, so a wave
// reads 64 x 16 contiguous bytes (fp32) per load instruction.  The block
// maximum is a 3-step xor-shuffle reduction inside each group of eight; the
// high-nibble codes of elements 16..31 (lanes 4..7) are shuffled down onto
// lanes 0..3, which then own four finished code bytes each.  The kernel is
// HBM-bound: it reads 4 (fp32) or 2 (fp16) bytes and writes 0.5625 bytes per
// weight.  Division is the IEEE-correct fp32 division: the library is built
// without fast-math.
#include "q4_internal.hpp"

namespace q4 {
namespace {

template <typename T>
struct Load4;

template <>
struct Load4<float> {
  static __device__ __forceinline__ void run(const float* p, float v[4]) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
};

template <>
struct Load4<half_t> {
  static __device__ __forceinline__ void run(const half_t* p, float v[4]) {
    const half4_t t = *reinterpret_cast<const half4_t*>(p);
    v[0] = static_cast<float>(t[0]); v[1] = static_cast<float>(t[1]);
    v[2] = static_cast<float>(t[2]); v[3] = static_cast<float>(t[3]);
  }
};

template <typename T>
__global__ __launch_bounds__(256) void quantize_kernel(const T* __restrict__ w,
                                                       uint8_t* __restrict__ out,
                                                       int64_t nblocks) {
  const int part = threadIdx.x & 7;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 3);
  // Grid-stride over blocks; the eight lanes of a group always share `blk`,
  // so they enter and leave the loop together.
  for (int64_t blk = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 3;
       blk < nblocks; blk += stride) {
  float v[4];
  Load4<T>::run(w + blk * kQK + part * 4, v);

  // Largest magnitude inside this lane, first index on ties.
  float best = v[0];
  float bmag = fabsf(v[0]);
  int bidx = part * 4;
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    const float a = fabsf(v[i]);
    if (a > bmag) { bmag = a; best = v[i]; bidx = part * 4 + i; }
  }
  // Across the eight lanes of the block; the combine is symmetric so every
  // lane ends with the same (value, index).
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    const float ob = __shfl_xor(best, off, 8);
    const int oi = __shfl_xor(bidx, off, 8);
    const float om = fabsf(ob);
    if (om > bmag || (om == bmag && oi < bidx)) { best = ob; bmag = om; bidx = oi; }
  }

  // The quotient is exact in fp32 (a power-of-two scaling), then rounded once
  // to fp16.  The empty asm keeps the compiler from fusing the two steps into a
  // mixed-precision fma with a +0 addend, which would turn a -0 scale into +0
  // (an all +0 block must get d = fp16(+0 / -8) = -0).
  float t = best / -8.0f;
  asm volatile("" : "+v"(t));
  const half_t dh = static_cast<half_t>(t);
  const float D = static_cast<float>(dh);

  uint32_t nib = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int q = 8;
    if (D != 0.0f) {
      const float u = v[i] / D;
      const float t = u + 8.5f;
      q = static_cast<int>(truncf(t));
      q = q < 0 ? 0 : (q > 15 ? 15 : q);
    }
    nib |= static_cast<uint32_t>(q) << (8 * i);
  }
  // Lane p (< 4) holds low nibbles of code bytes 4p..4p+3; lane p+4 holds the
  // matching high nibbles (elements 16 + 4p ..).
  const uint32_t hi = __shfl_down(nib, 4, 8);
  uint8_t* ob = out + blk * kBlockBytes;
  if (part < 4) {
    const uint32_t bytes = nib | (hi << 4);
    uint16_t* dst = reinterpret_cast<uint16_t*>(ob + 2 + 4 * part);  // 2-byte aligned
    dst[0] = static_cast<uint16_t>(bytes & 0xFFFFu);
    dst[1] = static_cast<uint16_t>(bytes >> 16);
  }
  if (part == 0) {
    *reinterpret_cast<uint16_t*>(ob) = __builtin_bit_cast(uint16_t, dh);
  }
  }
}

}  // namespace

hipError_t launch_quantize(const void* w, DType wt, int64_t n, int64_t k,
                           uint8_t* packed, hipStream_t s) {
  const int64_t nblocks = n * (k / kQK);
  const int64_t groups = (nblocks * 8 + 255) / 256;
  const dim3 grid(static_cast<unsigned>(groups < 65536 ? groups : 65536));
  const dim3 block(256);
  if (wt == DType::F32) {
    const float* p = static_cast<const float*>(w);
    void* argv[] = {&p, &packed, const_cast<int64_t*>(&nblocks)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_kernel<float>),
                           grid, block, argv, 0, s);
  }
  const half_t* p = static_cast<const half_t*>(w);
  void* argv[] = {&p, &packed, const_cast<int64_t*>(&nblocks)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_kernel<half_t>),
                         grid, block, argv, 0, s);
}

}  // namespace q4
