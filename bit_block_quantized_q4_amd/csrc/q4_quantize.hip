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
// maximum is a 3-step DPP reduction inside each group of eight; the
// high-nibble codes of elements 16..31 (lanes 4..7) are moved down onto
// lanes 0..3, which then own four finished code bytes each.  The kernel
// reads 4 (fp32) or 2 (fp16, bf16; both widened exactly to fp32) bytes and
// writes 0.5625 bytes per weight.  The
// codes follow the correctly rounded fp32 division exactly: a reciprocal with
// one residual step decides every code whose t is not within 2^-16 of an
// integer, the rest redo the IEEE division (the library is built without
// fast-math).
#include "q4_internal.hpp"

namespace q4 {
namespace {

constexpr int kQuantUF32 = 4;  // blocks in flight per lane group (16-byte loads)
constexpr int kQuantUF16 = 2;  // (8-byte loads; the kernel is VALU-bound, so more
                                // workgroups beat more loads in flight: 8 -> 2 took
                                // 5120 x 5120 fp16 from 30.2 to 23.0 us)

template <typename T>
struct Load4;

// fp32 weights are read with non-temporal loads: each byte is read once, and
// keeping the 4-byte input out of the caches measured 4 % faster (5120 x 5120:
// 24.5 -> 23.4 us; 17408 x 5120: 74.2 -> 71.0 us).  The 2-byte inputs gain
// nothing from it (their kernel is bound by its arithmetic), so they keep
// ordinary loads.
template <>
struct Load4<float> {
  static __device__ __forceinline__ void run(const float* p, float v[4]) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
  }
};

template <>
struct Load4<bf16_t> {
  static __device__ __forceinline__ void run(const bf16_t* p, float v[4]) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t t = *reinterpret_cast<const u32x2_t*>(p);
    v[0] = bf16_bits_to_float(t[0] & 0xFFFFu); v[1] = bf16_bits_to_float(t[0] >> 16);
    v[2] = bf16_bits_to_float(t[1] & 0xFFFFu); v[3] = bf16_bits_to_float(t[1] >> 16);
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

// Lane exchange inside a group of eight (DPP, no LDS round trip).
constexpr int kDppXor1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppShl4 = 0x104;     // lane i reads lane i + 4 (row_shl:4)

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

// Keep the (value, index) of larger magnitude, the smaller index on a tie.
template <int CTRL>
__device__ __forceinline__ void amax_step(float& best, float& bmag, int& bidx) {
  const float ob = dpp_f<CTRL>(best);
  const int oi = dpp_i<CTRL>(bidx);
  const float om = fabsf(ob);
  if (om > bmag || (om == bmag && oi < bidx)) { best = ob; bmag = om; bidx = oi; }
}

// Code q = min(15, trunc(fl(fl(x / D) + 8.5))) (negative truncations clamp to
// 0).  Fast path: r ~ 1/D (v_rcp_f32, 1 ulp), u = x r refined by one
// residual step e = fma(-u, D, x), u += e r, which leaves u within 2 ulp of
// the correctly rounded quotient (|u| <= 12 here, so 2^-19), and t = u + 8.5
// within 2^-18 of the rule's t.  Only a t within 2^-16 of an integer can
// truncate differently; those lanes redo the correctly rounded division.
__device__ __forceinline__ int code_of(float x, float D, float r) {
  float u = x * r;
  const float e = fmaf(-u, D, x);
  u = fmaf(e, r, u);
  float t = u + 8.5f;
  if (fabsf(t - __builtin_rintf(t)) < 0x1p-16f) {
    const float ue = x / D;
    asm volatile("" : "+v"(t));
    t = ue + 8.5f;
  }
  const int q = static_cast<int>(t);  // truncation
  return q < 0 ? 0 : (q > 15 ? 15 : q);
}

// One block: the eight lanes of a group share `blk` and hold its elements
// 4p .. 4p + 3 in v.
__device__ __forceinline__ void quantize_block(int64_t blk, int part, const float (&v)[4],
                                               uint8_t* __restrict__ out) {
  // Largest magnitude inside this lane, first index on ties.
  float best = v[0];
  float bmag = fabsf(v[0]);
  int bidx = part * 4;
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    const float a = fabsf(v[i]);
    if (a > bmag) { bmag = a; best = v[i]; bidx = part * 4 + i; }
  }
  // Across the eight lanes: both quads, then the other quad (the mirror pairs
  // lanes whose quads already agree), so every lane ends with the same pair.
  amax_step<kDppXor1>(best, bmag, bidx);
  amax_step<kDppXor2>(best, bmag, bidx);
  amax_step<kDppHalfMirror>(best, bmag, bidx);

  // The quotient is exact in fp32 (a power-of-two scaling), then rounded once
  // to fp16.  The empty asm keeps the compiler from fusing the two steps into a
  // mixed-precision fma with a +0 addend, which would turn a -0 scale into +0
  // (an all +0 block must get d = fp16(+0 / -8) = -0).
  float t = best / -8.0f;
  asm volatile("" : "+v"(t));
  const half_t dh = static_cast<half_t>(t);
  const float D = static_cast<float>(dh);

  uint32_t nib = 0x08080808u;  // every q is 8 when d is zero
  if (D != 0.0f) {
    const float r = __builtin_amdgcn_rcpf(D);
    nib = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) nib |= static_cast<uint32_t>(code_of(v[i], D, r)) << (8 * i);
  }
  // Lane p (< 4) holds low nibbles of code bytes 4p..4p+3; lane p+4 holds the
  // matching high nibbles (elements 16 + 4p ..).
  const uint32_t hi = static_cast<uint32_t>(dpp_i<kDppShl4>(static_cast<int>(nib)));
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

// Each group of eight lanes takes U blocks per sweep, blk0 + u * stride, and
// issues all U loads before quantising any: one load in flight per lane would
// leave about 32 KB in flight per CU, which at HBM latency caps the stream
// near 4 TB/s.
template <typename T, int U>
__global__ __launch_bounds__(256) void quantize_kernel(const T* __restrict__ w,
                                                       uint8_t* __restrict__ out,
                                                       int64_t nblocks) {
  const int part = threadIdx.x & 7;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 3);
  // The eight lanes of a group always share their blocks, so they take every
  // branch together (the shuffles stay within active groups).
  for (int64_t blk0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 3;
       blk0 < nblocks; blk0 += U * stride) {
    float v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t blk = blk0 + u * stride;
      if (blk < nblocks) Load4<T>::run(w + blk * kQK + part * 4, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t blk = blk0 + u * stride;
      if (blk < nblocks) quantize_block(blk, part, v[u], out);
    }
  }
}

}  // namespace

hipError_t launch_quantize(const void* w, DType wt, int64_t n, int64_t k,
                           uint8_t* packed, hipStream_t s) {
  const int64_t nblocks = n * (k / kQK);
  const int U = wt == DType::F32 ? kQuantUF32 : kQuantUF16;
  const int64_t groups = (nblocks + 32 * U - 1) / (32 * U);  // 32 blocks per workgroup per sweep
  const dim3 grid(static_cast<unsigned>(groups < 65535 ? groups : 65535));
  const dim3 block(256);
  if (wt == DType::F32) {
    const float* p = static_cast<const float*>(w);
    void* argv[] = {&p, &packed, const_cast<int64_t*>(&nblocks)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_kernel<float, kQuantUF32>),
                           grid, block, argv, 0, s);
  }
  if (wt == DType::BF16) {
    const bf16_t* p = static_cast<const bf16_t*>(w);
    void* argv[] = {&p, &packed, const_cast<int64_t*>(&nblocks)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_kernel<bf16_t, kQuantUF16>),
                           grid, block, argv, 0, s);
  }
  const half_t* p = static_cast<const half_t*>(w);
  void* argv[] = {&p, &packed, const_cast<int64_t*>(&nblocks)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_kernel<half_t, kQuantUF16>),
                         grid, block, argv, 0, s);
}

}  // namespace q4
