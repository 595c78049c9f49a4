// Device helpers shared by the libq4 kernels (gfx950).  Internal header.
#pragma once

#include "q4_internal.hpp"

namespace q4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Bit patterns used by the unpack.  They are kept in registers (see
// UnpackConsts) because VOP3 instructions cannot encode literals on gfx9, and
// v_and_or_b32 needs all three operands in registers.
struct UnpackConsts {
  uint32_t mask_lo, mask_hi;  // 0x000F000F, 0x00F000F0
  uint32_t exp_lo, exp_hi;    // fp16 1024 (0x6400) and 64 (0x5400) in both halves
};

__device__ __forceinline__ UnpackConsts make_unpack_consts() {
  UnpackConsts k{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
  asm volatile("" : "+s"(k.mask_lo), "+s"(k.mask_hi), "+v"(k.exp_lo), "+v"(k.exp_hi));
  return k;
}

// Exact fp16 (q - 8) for the eight codes of bytes c0..c3 taken from the 8-byte
// LDS window {w1:w0} at byte offset O, in operand order
// (e0, e1, e2, e3, e16, e17, e18, e19) relative to the lane's element base:
// low nibble q becomes fp16 1024 + q and high nibble q becomes 64 + q (the
// nibble lands in the low mantissa bits of a fixed exponent), then one exact
// packed subtraction of 1032 / 72 leaves q - 8.
template <int O>
__device__ __forceinline__ half8_t unpack8(uint32_t w0, uint32_t w1, const UnpackConsts& k) {
  constexpr uint32_t sel01 = (O + 0) | (0x0cu << 8) | ((O + 1u) << 16) | (0x0cu << 24);
  constexpr uint32_t sel23 = (O + 2) | (0x0cu << 8) | ((O + 3u) << 16) | (0x0cu << 24);
  const uint32_t t01 = __builtin_amdgcn_perm(w1, w0, sel01);  // [c0, 0, c1, 0]
  const uint32_t t23 = __builtin_amdgcn_perm(w1, w0, sel23);  // [c2, 0, c3, 0]
  const half2_t lo01 = __builtin_bit_cast(half2_t, (t01 & k.mask_lo) | k.exp_lo);
  const half2_t lo23 = __builtin_bit_cast(half2_t, (t23 & k.mask_lo) | k.exp_lo);
  const half2_t hi01 = __builtin_bit_cast(half2_t, (t01 & k.mask_hi) | k.exp_hi);
  const half2_t hi23 = __builtin_bit_cast(half2_t, (t23 & k.mask_hi) | k.exp_hi);
  const half2_t klo = {static_cast<half_t>(-1032.0f), static_cast<half_t>(-1032.0f)};
  const half2_t khi = {static_cast<half_t>(-72.0f), static_cast<half_t>(-72.0f)};
  const half2_t a = lo01 + klo, b = lo23 + klo, c = hi01 + khi, d = hi23 + khi;
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, a);
  r[1] = __builtin_bit_cast(uint32_t, b);
  r[2] = __builtin_bit_cast(uint32_t, c);
  r[3] = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(half8_t, r);
}

typedef __attribute__((address_space(3))) void* lptr_t;

// 16-byte global -> LDS copy for every active lane: lane l's bytes land at
// lds + 16 * l (the LDS base, held in M0, must be uniform across the wave).
// Issued as inline asm so that the compiler tracks no LDS-DMA writes of its
// own: every wait on these copies is the explicit wait_vm below.
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lptr_t)(lds)));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base) : "memory");
}
// As dma16 with the non-temporal hint (nt): for bytes read once per launch,
// the packed weights of the decode GEMV, which are then not kept in the
// caches in place of data that is read again (the activations).
__device__ __forceinline__ void dma16_nt(const void* src, void* lds) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lptr_t)(lds)));
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(base) : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
// Emitted through the s_waitcnt builtin (not inline asm) so that the
// compiler's own wait tracking knows the counter has drained and does not
// add a later wait that would also cover copies issued after this point.
// The fence keeps LDS reads of the awaited data below it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4] = 7, lgkmcnt[11:8] = 15
  constexpr int kImm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(kImm);
  asm volatile("" ::: "memory");
}

// As wait_vm, and also until every LDS operation of this wave has completed.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int kImm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4);
  __builtin_amdgcn_s_waitcnt(kImm);
  asm volatile("" ::: "memory");
}

// Wait until every LDS operation of this wave has completed (vector-memory
// copies may stay in flight).
__device__ __forceinline__ void wait_lgkm0() {
  // vmcnt at its maximum (63), expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
  asm volatile("" ::: "memory");
}

// As wait_vm / wait_vm_lgkm0 for a run-time count n <= MAXN (a chain of
// uniform compares choosing the immediate).
template <int MAXN>
__device__ __forceinline__ void wait_vm_upto(int n) {
  if constexpr (MAXN == 0) {
    wait_vm<0>();
  } else {
    if (n >= MAXN) {
      wait_vm<MAXN>();
      return;
    }
    wait_vm_upto<MAXN - 1>(n);
  }
}
template <int MAXN>
__device__ __forceinline__ void wait_vm_lgkm0_upto(int n) {
  if constexpr (MAXN == 0) {
    wait_vm_lgkm0<0>();
  } else {
    if (n >= MAXN) {
      wait_vm_lgkm0<MAXN>();
      return;
    }
    wait_vm_lgkm0_upto<MAXN - 1>(n);
  }
}

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// Register loads the compiler does not track (inline asm): the caller must
// drain them with wait_vm and tie the results to that wait (see tie_after)
// before reading them.  Used where copies into LDS and register loads share
// one explicit wait, so that no compiler-inserted wait drains both.
__device__ __forceinline__ u32x3 load_dwordx3_untracked(const void* p) {
  u32x3 v;
  asm volatile("global_load_dwordx3 %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}
__device__ __forceinline__ uint32_t load_ushort_untracked(const void* p) {
  uint32_t v;
  asm volatile("global_load_ushort %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}
__device__ __forceinline__ u32x4 load_dwordx4_untracked(const void* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}
__device__ __forceinline__ uint32_t load_dword_untracked(const void* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Scalar-base 16-byte global -> LDS copy: a 64-bit wave-uniform base (SGPR
// pair) plus a 32-bit per-lane byte offset; lane l's 16 bytes land at LDS byte
// address lds + 16 * l (lds uniform, held in M0).  Untracked like dma16.
__device__ __forceinline__ void dma16_sbase(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// As dma16_sbase with the non-temporal hint (see dma16_nt).
__device__ __forceinline__ void dma16_sbase_nt(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lptr_t)(p)));
}

// Make `v` depend on a point after an explicit wait, so its readers cannot be
// scheduled above that wait.
template <typename T>
__device__ __forceinline__ void tie_after(T& v) {
  asm volatile("" : "+v"(v));
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Whether any thread of the workgroup passed `flag`, through one word of the
// kernel's own LDS (`word`, free at this point: no thread reads or writes it
// after the first barrier until it returns).  Every thread must call it.  The
// barriers also order the global stores made before it ahead of later
// stores to the same outputs.  (__syncthreads_or would add static LDS, which
// kernels that take all 160 KB as dynamic LDS cannot launch with.)
__device__ __forceinline__ bool workgroup_any_flag(bool flag, uint32_t* word) {
  __syncthreads();
  if (threadIdx.x == 0) *word = 0u;
  __syncthreads();
  if (flag) *word = 1u;  // every writer writes the same value
  __syncthreads();
  return *word != 0u;
}

// Rows row0 .. row0 + nrows - 1 of y = x . dequant(W)^T for bf16 activations
// on the exact route: x widened exactly to fp32, (q - 8) and d applied in
// fp32 per block, fp32 FMAs, and a fixed-order reduction across the wave.
// The NW waves of the workgroup take rows w, w + NW, ...; lane l takes blocks
// l, l + 64, ....  The decode kernels use it where their fp16 conversion of
// bf16 activations was inexact (values beyond fp16's range or off its
// subnormal grid); it overwrites those rows' outputs.
template <int NW>
__device__ __forceinline__ void gemv_exact_rows_bf16(const uint16_t* x, const uint8_t* W, void* y,
                                                     int y_f16, int m, int64_t n, int64_t k,
                                                     int64_t row0, int nrows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t nb = k / kQK;
  const int64_t rb = nb * kBlockBytes;
#pragma unroll 1
  for (int r = wave; r < nrows; r += NW) {
    const int64_t row = row0 + r;
    const uint8_t* wr = W + row * rb;
#pragma unroll 1
    for (int mi = 0; mi < m; ++mi) {
      const uint16_t* xr = x + static_cast<int64_t>(mi) * k;
      float acc = 0.0f;
      for (int64_t b = lane; b < nb; b += kWave) {
        const uint8_t* blk = wr + b * kBlockBytes;
        const float d = half_bits_to_float(static_cast<uint16_t>(blk[0] | (blk[1] << 8)));
        const uint16_t* xb = xr + b * kQK;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int c = blk[2 + j];
          s = __builtin_fmaf(bf16_bits_to_float(xb[j]), static_cast<float>((c & 0xF) - 8), s);
          s = __builtin_fmaf(bf16_bits_to_float(xb[j + 16]), static_cast<float>((c >> 4) - 8), s);
        }
        acc = __builtin_fmaf(d, s, acc);
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (lane == 0) {
        const int64_t o = static_cast<int64_t>(mi) * n + row;
        if (y_f16) static_cast<half_t*>(y)[o] = static_cast<half_t>(acc);
        else static_cast<float*>(y)[o] = acc;
      }
    }
  }
}


}  // namespace q4
