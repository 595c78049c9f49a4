// Q4_0 prefill GEMM for gfx950: y[m][n] = x[m][k] . dequant(W)^T on fp16 MFMA.
//
// The GPU path from Q4_0 weights onto matrix cores of the vertical-disaggregation page
// (section "Every cycle counts: custom kernels"): long prompts are dense
// computation, so weights are dequantised once per workgroup to fp16
// w = (q - 8) * d (one rounding) and contracted with the fp16 activations on
// v_mfma_f32_32x32x16_f16 with fp32 accumulation.  Every output is summed in a
// fixed order (k order within one lane; for slice-K tiles the four slice
// partials then in wave order; for split-K tails the splits in split order),
// so results are bit-reproducible.
//
// Kernels
// -------
//   - gemm_mfma_kernel (k % 64 == 0): a BM x BN output tile per workgroup
//     (256 x 256 with 8 waves, each 128 x 64, for m >= 1024; else 128 x 128
//     with 4 waves of 64 x 64), k steps of 64 (two Q4_0 blocks), two LDS
//     stages.  Activations arrive by direct global->LDS copies
//     (global_load_lds_dwordx4) into an XOR swizzle (piece c of row r at
//     r*8 + (c ^ key(r)), key(r) = (r & 7) ^ ((r >> 3) & 1)) under which the
//     16-byte operand reads have no bank conflicts.  Each
//     thread owns weight units (one whole block of one row), loads them two
//     steps ahead, dequantises them with byte permutes, the 1024+q / 64+q
//     exponent trick, an exact packed subtraction and one packed multiply by
//     d, and writes them into the other stage in the same swizzle, interleaved
//     with the step's matrix products.  One barrier per step.
//   - gemm_slicek_kernel (m < 1024, k % 256 == 0, k >= 1024): 128 x 128 tiles
//     whose four waves each own the whole tile for one k16 slice of every
//     step, with packed weights copied into LDS and dequantised in registers
//     by the one wave that uses them; see its own comment.
//   - gemm_tile_kernel: the generic LDS-tiled kernel for k % 64 != 0.
//   - gemm_exact_kernel: the exact route (fp32 activations; see exact_tile128).
// Launches run whole rounds of tiles on the compute units; a partial round's
// columns run the same tiles with K split across workgroups (fp32 partials,
// then splitk_reduce_kernel in split order).
//
// The fp16 tiles are exact up to fp32 summation only while every dequantised
// weight and every activation is an fp16 value.  A block scale |d| > 8188
// breaks the first (its largest element, code 0, dequantises to 8 |d| >
// 65504, i.e. to +-inf), and bf16 activations outside fp16's range or off
// its subnormal grid break the second (the bf16 staging pass writes such a
// row as NaN).  Either makes the tile's fp32 accumulators non-finite, so
// every fp16 kernel checks its accumulators once at the end and a workgroup
// that finds a non-finite one recomputes its tile (and K range) on the exact
// route from the original activations.  In-domain results are finite, so the
// check never fires on them.
#include <initializer_list>

#include "q4_device.hpp"

namespace q4 {
namespace {

template <int V>
struct IC {
  static constexpr int value = V;
};

constexpr int BM = 128;       // rows of x per workgroup
constexpr int BN = 128;       // output features per workgroup
constexpr int BK = kQK;       // one Q4_0 block per k step
constexpr int LDK = BK + 8;   // padded LDS row (halves)

// ------------------------------------------------------------------ exact route
//
// y = sum over blocks of sum_j x[j] (q_j - 8) d with the activations widened
// exactly to fp32 (from fp32, fp16 or bf16) and the weights dequantised
// exactly to fp32, contracted on v_mfma_f32_32x32x2_f32 (fp32 operands, fp32
// accumulation): every product is formed from the exact operands, so the
// error is fp32 summation error relative to sum |x w|, for every in-domain
// input.  It is several times slower than the fp16 tiles.
constexpr int kExLd = 17;                        // floats per LDS row (16 k + 1 pad)
constexpr int kExLdsBytes = 2 * 128 * kExLd * 4;  // 17408

__device__ __forceinline__ float load_x_f32(const void* x, DType xt, int64_t i) {
  if (xt == DType::F32) return static_cast<const float*>(x)[i];
  if (xt == DType::F16) return static_cast<float>(static_cast<const half_t*>(x)[i]);
  return bf16_bits_to_float(static_cast<const uint16_t*>(x)[i]);
}

// One 128 x 128 output tile: activation rows r0 .. r0 + 127 (of m) against
// weight rows (output columns) c0 .. c0 + 127 (of n), over the Q4_0 blocks
// b0 .. b1 - 1 of K; y holds the tile's outputs at row stride ldy (final
// outputs or fp32 split-K partials).  NTH threads (4 or 8 waves) stage each
// half block (16 k) of x and of the dequantised weights in LDS; the waves
// split the tile 2 x 2 (64 x 64 each, 2 x 2 products of 32 x 32) or, with
// eight waves, 4 x 2 (32 x 64 each, 1 x 2 products), which keeps the
// fallback's registers few where it is inlined into a large kernel.
template <int NTH, typename YT>
__device__ __forceinline__ void exact_tile128(const void* x, DType xt, int64_t ldx, const uint8_t* W,
                                              int64_t rb, YT* y, int64_t ldy, int64_t m, int64_t n,
                                              int64_t r0, int64_t c0, int64_t b0, int64_t b1,
                                              float* lds) {
  static_assert(NTH == 256 || NTH == 512, "four or eight waves");
  constexpr int WVM = NTH == 512 ? 4 : 2;  // waves along the rows
  constexpr int TI = 4 / WVM;              // 32-row products per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  float* As = lds;
  float* Bs = lds + 128 * kExLd;
  float16_t acc[TI][2];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
#pragma unroll 1
  for (int64_t b = b0; b < b1; ++b) {
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      __syncthreads();  // the previous half's operand reads are done
      for (int e = tid; e < 128 * 16; e += NTH) {
        const int r = e >> 4, j = e & 15;
        const int64_t gr = r0 + r, gc = c0 + r;
        As[r * kExLd + j] = gr < m ? load_x_f32(x, xt, gr * ldx + kQK * b + 16 * h + j) : 0.0f;
        float w = 0.0f;
        if (gc < n) {
          const uint8_t* blk = W + gc * rb + b * kBlockBytes;
          const float d = half_bits_to_float(static_cast<uint16_t>(blk[0] | (blk[1] << 8)));
          const int q = (blk[2 + j] >> (4 * h)) & 0xF;
          w = static_cast<float>(q - 8) * d;
        }
        Bs[r * kExLd + j] = w;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int kc = 2 * kk + (lane >> 5);  // lane l supplies k = l / 32 of the pair
        float a[TI], bv[2];
#pragma unroll
        for (int i = 0; i < TI; ++i)
          a[i] = As[(wm * 32 * TI + 32 * i + (lane & 31)) * kExLd + kc];
#pragma unroll
        for (int j = 0; j < 2; ++j) bv[j] = Bs[(wn * 64 + 32 * j + (lane & 31)) * kExLd + kc];
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
  }
  // 32 x 32 accumulator layout: lane l holds column l % 32; register r holds
  // row 8 (r / 4) + 4 (l / 32) + r % 4.
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = r0 + wm * 32 * TI + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = c0 + wn * 64 + 32 * j + (lane & 31);
        if (row < m && col < n) y[row * ldy + col] = static_cast<YT>(acc[i][j][r]);
      }
}

// A BMT x BNT tile (multiples of 128) on the exact route, 128 x 128 at a time.
template <int NTH, int BMT, int BNT, typename YT>
__device__ __forceinline__ void exact_tile(const void* x, DType xt, int64_t ldx, const uint8_t* W, int64_t rb,
                           YT* y, int64_t ldy, int64_t m, int64_t n, int64_t m0, int64_t n0,
                           int64_t b0, int64_t b1, float* lds) {
#pragma unroll 1
  for (int ti = 0; ti < BMT / 128; ++ti)
#pragma unroll 1
    for (int tj = 0; tj < BNT / 128; ++tj)
      exact_tile128<NTH, YT>(x, xt, ldx, W, rb, y, ldy, m, n, m0 + 128 * ti, n0 + 128 * tj, b0, b1,
                             lds);
}

// Exact route as a kernel: one 128 x 128 tile per workgroup over all of K
// (fp32 activations).
template <typename YT>
__global__ __launch_bounds__(256) void gemm_exact_kernel(const void* __restrict__ x, int xt,
                                                         const uint8_t* __restrict__ W,
                                                         YT* __restrict__ y, int64_t m, int64_t n,
                                                         int64_t k) {
  __shared__ __attribute__((aligned(16))) float lds[kExLdsBytes / 4];
  exact_tile128<256, YT>(x, static_cast<DType>(xt), k, W, (k / kQK) * kBlockBytes, y, n, m, n,
                         static_cast<int64_t>(blockIdx.y) * 128, static_cast<int64_t>(blockIdx.x) * 128,
                         0, k / kQK, lds);
}

template <typename YT>
__global__ __launch_bounds__(256) void gemm_tile_kernel(
    const half_t* __restrict__ x, const uint8_t* __restrict__ W, YT* __restrict__ y,
    int64_t m, int64_t n, int64_t k, const void* __restrict__ xe, int xet) {
  // xe / xet: the original activations, for the exact route.
  constexpr int kTileLds = 2 * BM * LDK * 2 > kExLdsBytes ? 2 * BM * LDK * 2 : kExLdsBytes;
  __shared__ __attribute__((aligned(16))) uint8_t tsm[kTileLds];
  half_t (*As)[LDK] = reinterpret_cast<half_t (*)[LDK]>(tsm);
  half_t (*Bs)[LDK] = reinterpret_cast<half_t (*)[LDK]>(tsm + BM * LDK * 2);

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
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = acc[i][j][r];
        bad |= !__builtin_isfinite(v);
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < m && col < n) y[row * n + col] = static_cast<YT>(v);
      }
  if (workgroup_any_flag(bad, reinterpret_cast<uint32_t*>(tsm)))
    exact_tile128<256, YT>(xe, static_cast<DType>(xet), k, W, nb * kBlockBytes, y, n, m, n, m0, n0,
                           0, nb, reinterpret_cast<float*>(tsm));
}


// ------------------------------------------------------------------ tiled

constexpr int kBK = 64;            // k per step: two Q4_0 blocks
constexpr int kRowBytes16 = 128;   // one tile row of 64 fp16 = 8 pieces of 16 bytes

// Swizzle key of LDS row r (128-byte rows of eight 16-byte pieces): piece c
// of row r sits at r * 8 + (c ^ key(r)).  Sixteen consecutive rows reading
// one piece column land in sixteen distinct 16-byte bank groups of a 256-byte
// bank window (rows r and r + 8 differ in the key's low bit), and any eight
// consecutive rows in eight distinct groups of a 128-byte window.
__device__ __forceinline__ int swz_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ swz_key(r)); }

// One weight unit: one block of a row (scale and 16 code bytes) as the
// 20-byte aligned window w0..w4 that contains it.
struct WUnit {
  u32x4 w;     // w0 .. w3
  uint32_t w4;
};

template <int BM, int BN, int WVM, int WVN, typename YT>
__global__ __launch_bounds__(WVM * WVN * 64, 1) void gemm_mfma_kernel(
    const half_t* __restrict__ x, const uint8_t* __restrict__ W, YT* __restrict__ y,
    int64_t m, int64_t n, int64_t k, int64_t ldy, int kps, int64_t zstride,
    const void* __restrict__ xe, int xet) {
  // k: full K (row strides).  Workgroups with blockIdx.z = z take the K steps
  // z kps .. min((z + 1) kps, k / 64) - 1 and write y + z zstride (a split-K
  // partial when gridDim.z > 1).  xe / xet: the original activations, for
  // the exact route.
  constexpr int NTH = WVM * WVN * 64;       // threads
  constexpr int WM = BM / WVM, WN = BN / WVN;  // wave tile
  constexpr int TM = WM / 32, TN = WN / 32; // 32 x 32 products per wave
  constexpr int A_STAGE = BM * kRowBytes16;
  constexpr int B_STAGE = BN * kRowBytes16;
  constexpr int STAGE = A_STAGE + B_STAGE;
  constexpr int A_COPIES = BM * 8 / NTH;    // 16-byte copies per thread per step
  constexpr int UNITS = BN * 2 / NTH;       // weight units (blocks) per thread per step
  static_assert(A_COPIES >= 1 && UNITS >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WVN, wn = wave % WVN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t rb = (k / kQK) * kBlockBytes;
  const int ks0 = static_cast<int>(blockIdx.z) * kps;
  const int nks_all = static_cast<int>(k / kBK);
  const int nks = nks_all - ks0 < kps ? nks_all - ks0 : kps;
  const uint8_t* const W0 = W;
  x += static_cast<int64_t>(ks0) * kBK;
  W += static_cast<int64_t>(ks0) * 2 * kBlockBytes;
  y += static_cast<int64_t>(blockIdx.z) * zstride;

  // Activation copies: copy i of this thread is LDS piece P = NTH i + tid
  // (row P / 8, swizzled column P % 8); the source column undoes the swizzle.
  const half_t* asrc[A_COPIES];
#pragma unroll
  for (int i = 0; i < A_COPIES; ++i) {
    const int P = NTH * i + tid;
    const int r = P >> 3;
    const int c = (P & 7) ^ swz_key(r);
    const int64_t row = m0 + r < m ? m0 + r : m - 1;
    asrc[i] = x + row * k + 8 * c;
  }
  auto issue_a = [&](int ks, int stage) {
    uint8_t* dst = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < A_COPIES; ++i)
      dma16(asrc[i] + static_cast<int64_t>(ks) * kBK, dst + (NTH * i + 64 * wave) * 16);
  };

  // Weight units: unit u of this thread is U = NTH u + tid: row U / 2, block
  // U % 2 of the step.  A step is 36 bytes of the row starting 4-byte aligned
  // (rows are 36-byte multiples here); block 0's window is its first 20
  // bytes, block 1's the last 20, so both stay inside the step.  In the window
  // the scale is at byte 2b and code byte c at 2 + 2b + c.
  const uint8_t* wsrc[UNITS];
  uint32_t sel_even[UNITS], sel_odd[UNITS], dshift[UNITS];
  int wrow[UNITS], wblk[UNITS];
#pragma unroll
  for (int u = 0; u < UNITS; ++u) {
    const int U = NTH * u + tid;
    const int r = U >> 1;
    const int b = U & 1;
    const int64_t row = n0 + r < n ? n0 + r : n - 1;
    wsrc[u] = W + row * rb + 16 * b;  // + 36 per step
    // code pair i' (bytes 8h + 2i', +1) sits at byte 2 + 2b + 2 (i' & 1) of
    // the dword pair {w[2h + i'/2 + 1] : w[2h + i'/2]}; selectors give [c, 0, c', 0]
    const uint32_t s0 = static_cast<uint32_t>(2 + 2 * b);
    const uint32_t s1 = s0 + 2;
    sel_even[u] = s0 | (0x0cu << 8) | ((s0 + 1) << 16) | (0x0cu << 24);
    sel_odd[u] = s1 | (0x0cu << 8) | ((s1 + 1) << 16) | (0x0cu << 24);
    dshift[u] = 16u * b;
    wrow[u] = r;
    wblk[u] = b;
  }
  // Untracked loads of the packed bytes of step ks (see load_dwordx4_untracked).
  struct Units {
    WUnit v[UNITS];
  };
  auto load_units = [&](int ks) {
    Units r;
#pragma unroll
    for (int u = 0; u < UNITS; ++u) {
      const uint8_t* src = wsrc[u] + static_cast<int64_t>(ks) * 2 * kBlockBytes;
      r.v[u].w = load_dwordx4_untracked(src);
      r.v[u].w4 = load_dword_untracked(src + 16);
    }
    return r;
  };
  auto tie_units = [&](Units& r) {
#pragma unroll
    for (int u = 0; u < UNITS; ++u) {
      tie_after(r.v[u].w);
      tie_after(r.v[u].w4);
    }
  };

  const UnpackConsts kc = make_unpack_consts();
  // Dequantise half h of unit u (16 weights) and store its two pieces into
  // `stage`: codes 8h .. 8h+7 give k 8h .. 8h+7 (low nibbles, piece 4b + h)
  // and k 16 + 8h .. (high nibbles, piece 4b + h + 2).
  auto dequant_half = [&](const WUnit& un, int u, int h, int stage) {
    const uint32_t w[5] = {un.w[0], un.w[1], un.w[2], un.w[3], un.w4};
    const uint32_t dbits = (w[0] >> dshift[u]) & 0xFFFFu;
    const half2_t d2 = __builtin_bit_cast(half2_t, dbits | (dbits << 16));
    const half2_t klo = {static_cast<half_t>(-1032.0f), static_cast<half_t>(-1032.0f)};
    const half2_t khi = {static_cast<half_t>(-72.0f), static_cast<half_t>(-72.0f)};
    uint8_t* bs = smem + stage * STAGE + A_STAGE;
    u32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t t = __builtin_amdgcn_perm(w[2 * h + i / 2 + 1], w[2 * h + i / 2],
                                               (i & 1) ? sel_odd[u] : sel_even[u]);
      const half2_t ql = __builtin_bit_cast(half2_t, (t & kc.mask_lo) | kc.exp_lo) + klo;
      const half2_t qh = __builtin_bit_cast(half2_t, (t & kc.mask_hi) | kc.exp_hi) + khi;
      lo[i] = __builtin_bit_cast(uint32_t, ql * d2);
      hi[i] = __builtin_bit_cast(uint32_t, qh * d2);
    }
    *reinterpret_cast<u32x4*>(bs + swz(wrow[u], 4 * wblk[u] + h) * 16) = lo;
    *reinterpret_cast<u32x4*>(bs + swz(wrow[u], 4 * wblk[u] + h + 2) * 16) = hi;
  };

  float16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Every vector-memory operation in the loop is untracked by the compiler
  // (LDS copies and register loads); each step ends with one explicit drain.
  // Prologue: stage 0 complete, packed weights of step 1 in registers.
  issue_a(0, 0);
  {
    Units u0 = load_units(0);
    wait_vm<0>();
    tie_units(u0);
#pragma unroll
    for (int u = 0; u < UNITS; ++u) {
      dequant_half(u0.v[u], u, 0, 0);
      dequant_half(u0.v[u], u, 1, 0);
    }
  }
  Units nxt = load_units(nks > 1 ? 1 : 0);
  wait_vm<0>();
  tie_units(nxt);
  __syncthreads();

  const int arow = wm * WM + (lane & 31);
  const int brow = wn * WN + (lane & 31);
  const int kg = lane >> 5;

  // Operand fragments of k16 sub-step kk of a stage (lane: row arow / brow,
  // 8 k-values 8 kg .. 8 kg + 7 of the sub-step).
  auto read_frags = [&](const uint8_t* as, int kk, half8_t (&af)[TM], half8_t (&bf)[TN]) {
    const uint8_t* bs = as + A_STAGE;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = *reinterpret_cast<const half8_t*>(as + swz(arow + 32 * i, 2 * kk + kg) * 16);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bf[j] = *reinterpret_cast<const half8_t*>(bs + swz(brow + 32 * j, 2 * kk + kg) * 16);
  };
  // Interleave the matrix products of a sub-step with the next sub-step's
  // operand reads and the dequantisation (one MFMA, one LDS read, two VALU).
  auto interleave = [](auto with_reads) {
    constexpr bool R = decltype(with_reads)::value;
#pragma unroll
    for (int i = 0; i < TM * TN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (R && i < TM + TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
    }
  };

  if constexpr (TM * TN <= 4) {
    // Small wave tiles (one wave per SIMD): few products per k16 sub-step
    // cannot cover an LDS read, so all four sub-steps' fragments of a stage
    // are read right after its barrier and the products then run back to
    // back, with the dequantisation interleaved.
    half8_t fa[4][TM], fb[4][TN];
    auto read_all = [&](const uint8_t* as) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) read_frags(as, kk, fa[kk], fb[kk]);
    };
    auto interleave_valu = []() {
#pragma unroll
      for (int i = 0; i < TM * TN; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
      }
    };
    read_all(smem);
    for (int ks = 0; ks < nks; ++ks) {
      const int st = ks & 1;
      issue_a(ks + 1 < nks ? ks + 1 : ks, st ^ 1);
      const Units cur = nxt;
      nxt = load_units(ks + 2 < nks ? ks + 2 : nks - 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < UNITS; ++u)
          for (int h = 0; h < 2; ++h)
            if ((2 * u + h) % 4 == kk) dequant_half(cur.v[u], u, h, st ^ 1);
        interleave_valu();
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vm<0>();
      tie_units(nxt);
      __syncthreads();
      read_all(smem + (st ^ 1) * STAGE);
    }
  } else {
    half8_t af[2][TM], bf[2][TN];
    read_frags(smem, 0, af[0], bf[0]);
    for (int ks = 0; ks < nks; ++ks) {
      const int st = ks & 1;
      // Activations of step ks + 1 into the other stage (the last step copies
      // its own again: that stage is no longer read).
      issue_a(ks + 1 < nks ? ks + 1 : ks, st ^ 1);
      const Units cur = nxt;
      nxt = load_units(ks + 2 < nks ? ks + 2 : nks - 1);
      const uint8_t* as = smem + st * STAGE;
  #pragma unroll
      for (int kk = 0; kk < 4; ++kk) {  // 16-wide k sub-steps
        const int c = kk & 1;
        if (kk < 3) read_frags(as, kk + 1, af[c ^ 1], bf[c ^ 1]);
  #pragma unroll
        for (int i = 0; i < TM; ++i)
  #pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][i], bf[c][j], acc[i][j], 0, 0, 0);
        // The next step's weights (on the last step: a harmless rewrite of the
        // stage no longer read).
  #pragma unroll
        for (int u = 0; u < UNITS; ++u)
          for (int h = 0; h < 2; ++h)
            if ((2 * u + h) % 4 == kk) dequant_half(cur.v[u], u, h, st ^ 1);
        if (kk < 3) interleave(IC<true>{});
        else interleave(IC<false>{});
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vm<0>();
      tie_units(nxt);
      __syncthreads();
      read_frags(smem + (st ^ 1) * STAGE, 0, af[0], bf[0]);
    }
  }

  // 32x32 accumulator layout: lane l holds column l % 32; register r holds
  // row 8 * (r / 4) + 4 * (l / 32) + r % 4.  (Storing y transposed from
  // swapped operands, four columns per 8-byte store, measured slower: each
  // store then touches 32 rows.)
  bool bad = false;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = acc[i][j][r];
        bad |= !__builtin_isfinite(v);
        const int64_t row = m0 + wm * WM + 32 * i + 8 * (r / 4) + 4 * kg + (r & 3);
        const int64_t col = n0 + wn * WN + 32 * j + (lane & 31);
        if (row < m && col < n) y[row * ldy + col] = static_cast<YT>(v);
      }
  // A non-finite accumulator: this tile's outputs are rewritten on the exact route.
  if (workgroup_any_flag(bad, reinterpret_cast<uint32_t*>(smem)))
    exact_tile<NTH, BM, BN, YT>(xe, static_cast<DType>(xet), k, W0, rb, y, ldy, m, n, m0, n0,
                                2 * static_cast<int64_t>(ks0), 2 * static_cast<int64_t>(ks0 + nks),
                                reinterpret_cast<float*>(smem));
}

// ------------------------------------------------------------------ slice-K
//
// 128 x 128 output tile, four waves, k % 256 == 0.  Wave w owns the whole
// tile for the k16 slice w of every 64-wide k step: k 16w .. 16w+15, which is
// one nibble half (w & 1) of block w >> 1 of the step.  Every activation and
// weight element is therefore read from LDS by one wave only and dequantised
// once, and a wave's operand fragments per step are four of each (against
// eight for a 2 x 2 split of the tile).  The four partial tiles are summed in
// wave order at the end.
//
// Copies (global -> LDS, 16-byte pieces, issued by all waves):
//   - activations: a ring of six 64-wide k stages, stage of step ks = ks % 6,
//     refilled five steps ahead;
//   - packed weights: the 144 bytes of each row that cover four steps (256 k,
//     16-byte aligned because k % 256 == 0), a ring of three, refilled three
//     segments ahead.
// Per step: issue copies, read the next step's activation fragments and the
// raw weights of the step after, run this step's 16 matrix products
// interleaved with those reads and with the dequantisation of the next
// step's weights (read one step earlier, so no arithmetic waits on a fresh
// LDS read), then one barrier once the copies the next step reads have
// landed.
constexpr int kSkAStage = 128 * kRowBytes16;        // 16 KB
constexpr int kSkSeg = 4 * 2 * kBlockBytes;         // 144 packed bytes per row and 4 steps
constexpr int kSkWStage = 128 * kSkSeg;             // 18 KB
constexpr int kSkAStages = 6;
constexpr int kSkWOff = kSkAStages * kSkAStage;     // weight ring after the activation ring
constexpr int kSkLds = kSkWOff + 3 * kSkWStage;     // 150 KB
constexpr int kSkRedCol = 36;                       // floats per column of a partial (32 rows + pad)
static_assert(4 * 128 * kSkRedCol * 4 <= kSkLds, "reduction buffer");

template <typename YT>
__global__ __launch_bounds__(256, 1) void gemm_slicek_kernel(
    const half_t* __restrict__ x, const uint8_t* __restrict__ W, YT* __restrict__ y,
    int64_t m, int64_t n, int64_t k, int64_t ldy, int kps, int64_t zstride,
    const void* __restrict__ xe, int xet) {
  // k: full K (row strides).  Workgroups with blockIdx.z = z take the k steps
  // z kps .. min((z + 1) kps, k / 64) - 1 (kps % 4 == 0) and write y + z zstride.
  // xe / xet: the original activations, for the exact route.
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSkLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 5, lc = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 128;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 128;
  const int64_t rb = (k / kQK) * kBlockBytes;
  const int ks0 = static_cast<int>(blockIdx.z) * kps;
  const int nks_all = static_cast<int>(k / kBK);
  const int nks = nks_all - ks0 < kps ? nks_all - ks0 : kps;  // a multiple of 4
  const int nss = nks >> 2;
  const uint8_t* const W0 = W;
  x += static_cast<int64_t>(ks0) * kBK;
  W += static_cast<int64_t>(ks0) * 2 * kBlockBytes;
  y += static_cast<int64_t>(blockIdx.z) * zstride;

  // Copies take a wave-uniform base (the tile's first row at step ks, or its
  // first weight row at segment ss) plus a 32-bit per-lane byte offset.
  // Activation copy i of this thread: LDS piece P = 256 i + tid of a stage
  // (row P / 8, swizzled column P % 8).
  const uint32_t lds0 = lds_addr(smem);
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int P = 256 * i + tid;
    const int r = P >> 3;
    const int c = (P & 7) ^ swz_key(r);
    const int64_t rr = m0 + r < m ? r : m - 1 - m0;
    aoff[i] = static_cast<uint32_t>((rr * k + 8 * c) * 2);
  }
  const half_t* const xt = x + m0 * k;
  auto issue_a = [&](int ks, int stage) {
    const half_t* base = xt + static_cast<int64_t>(ks) * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16_sbase(aoff[i], base, lds0 + stage * kSkAStage + (256 * i + 64 * wave) * 16);
  };
  // Weight copy i of this thread: piece p of a weight stage (row p / 9, piece
  // p % 9 of its 144 bytes); 1152 pieces = four full rounds of 256 plus a
  // fifth in which each wave copies 32.
  uint32_t woff[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int p = i < 4 ? 256 * i + tid : 1024 + 32 * wave + lc;
    const int r = p / 9;
    const int c = p - 9 * r;
    const int64_t rr = n0 + r < n ? r : n - 1 - n0;
    woff[i] = static_cast<uint32_t>(rr * rb + 16 * c);
  }
  const uint8_t* const wt = W + n0 * rb;
  auto issue_w = [&](int ss, int buf) {
    const uint8_t* base = wt + static_cast<int64_t>(ss) * kSkSeg;
    const uint32_t dst = lds0 + kSkWOff + buf * kSkWStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_sbase(woff[i], base, dst + (256 * i + 64 * wave) * 16);
    if (lane < 32) dma16_sbase(woff[4], base, dst + (1024 + 32 * wave) * 16);
  };

  // This wave's share of a step: block b = w >> 1 of the step and its code
  // bytes 8h .. 8h + 7 (h = w & 1), both nibbles.  The k order inside a
  // matrix product is free as long as both operands follow it: lane (lc, kg)
  // takes the low nibbles (kg = 0, block elements 8h .. 8h + 7) or the high
  // nibbles (kg = 1, elements 16 + 8h ..) of those bytes, and its activation
  // fragment is the matching 8 halves, piece 4b + 2kg + h of the step.  Both
  // halves of the wave read the same weight bytes (one LDS broadcast): the
  // aligned 12-byte window at step byte 16b + 8h (code byte 8h + e at window
  // byte O + e, O = 2 + 2b) and the scale as the dword at 16b (its low half
  // for b = 0, high half for b = 1).
  const int b = wave >> 1, h = wave & 1;
  const uint32_t O = 2u + 2u * static_cast<uint32_t>(b);
  const uint32_t sel_a = O | (0x0cu << 8) | ((O + 1) << 16) | (0x0cu << 24);
  const uint32_t sel_b = (O + 2) | (0x0cu << 8) | ((O + 3) << 16) | (0x0cu << 24);
  const uint32_t nib_mask = kg ? 0x00F000F0u : 0x000F000Fu;
  const uint32_t nib_exp = kg ? 0x54005400u : 0x64006400u;  // fp16 64 + q / 1024 + q
  const half_t sub1 = static_cast<half_t>(kg ? -72.0f : -1032.0f);
  const half2_t nib_sub = {sub1, sub1};
  const uint32_t dshift = 16u * static_cast<uint32_t>(b);
  const int apiece = 4 * b + 2 * kg + h;

  struct Raw {
    uint32_t w[4][3];
    uint32_t d[4];
  };
  // Fragment reads from a lane base plus compile-time offsets (stage, buffer,
  // step within the segment, fragment).  Reads past the last step are of
  // valid LDS addresses and unused.
  const uint8_t* const abase = smem + swz(lc, apiece) * 16;  // + 32 i rows: swz(32 i + lc, apiece)
  const uint8_t* const wbase = smem + kSkWOff + lc * kSkSeg + 16 * b;
  auto read_a = [&](auto stage_c, half8_t (&fa)[4]) {
    constexpr int stage = decltype(stage_c)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[i] = *reinterpret_cast<const half8_t*>(abase + stage * kSkAStage + i * 4096);
  };
  auto read_w = [&](const uint8_t* wb, auto j_c, Raw& raw) {
    constexpr int off = 36 * decltype(j_c)::value;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint8_t* rp = wb + off + jj * 32 * kSkSeg;
      const uint32_t* win = reinterpret_cast<const uint32_t*>(rp + 8 * h);
      raw.w[jj][0] = win[0];
      raw.w[jj][1] = win[1];
      raw.w[jj][2] = win[2];
      raw.d[jj] = *reinterpret_cast<const uint32_t*>(rp);
    }
  };
  auto dequant = [&](const Raw& raw, half8_t (&fb)[4]) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t db = (raw.d[jj] >> dshift) & 0xFFFFu;
      const half2_t d2 = __builtin_bit_cast(half2_t, db | (db << 16));
      const uint32_t w0 = raw.w[jj][0], w1 = raw.w[jj][1], w2 = raw.w[jj][2];
      const uint32_t t[4] = {__builtin_amdgcn_perm(w1, w0, sel_a), __builtin_amdgcn_perm(w1, w0, sel_b),
                             __builtin_amdgcn_perm(w2, w1, sel_a), __builtin_amdgcn_perm(w2, w1, sel_b)};
      u32x4 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const half2_t v = __builtin_bit_cast(half2_t, (t[q] & nib_mask) | nib_exp) + nib_sub;
        r[q] = __builtin_bit_cast(uint32_t, v * d2);
      }
      fb[jj] = __builtin_bit_cast(half8_t, r);
    }
  };

  float16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Prologue: copies in the order the loop's waits assume (W0 A0 W1 A1 A2
  // A3 A4 W2, as if steps -5 .. -1 had run); once A0, W0 and A1 have landed:
  // step 0's operands and step 1's raw weights.
  const int last = nks - 1;
  issue_w(0, 0);
  issue_a(0, 0);
  issue_w(1 < nss - 1 ? 1 : nss - 1, 1);
  issue_a(1 < last ? 1 : last, 1);
  issue_a(2 < last ? 2 : last, 2);
  issue_a(3 < last ? 3 : last, 3);
  issue_a(4 < last ? 4 : last, 4);
  issue_w(2 < nss - 1 ? 2 : nss - 1, 2);
  wait_vm_lgkm0<17>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  half8_t fa[4], fb[4];
  Raw rc;  // raw weights of step ks + 1
  {
    Raw r0;
    read_a(IC<0>{}, fa);
    read_w(wbase, IC<0>{}, r0);
    read_w(wbase, IC<1>{}, rc);
    dequant(r0, fb);
  }
  // (step 0 refills stage 5, which nothing has read: no barrier needed here)

  // Step ks = 4 ss + j works on operands in registers and, for the steps
  // ahead, reads step ks + 1's activation fragments and step ks + 2's raw
  // weights and dequantises step ks + 1's.  Copies: A(ks + 5) into stage
  // (ks - 1) % 6, and at j = 3, after it, weight segment ss + 3 into buffer
  // ss % 3.  Both were last read a step before this one and those reads were
  // consumed (by step ks - 1's products, by this step's predecessor's
  // dequantisation) before the last barrier, so no wave waits for its LDS
  // reads at a barrier.  The wait is for A(ks + 2), which step ks + 1 reads:
  // issued at step ks - 3, it has the three later activation copies and
  // exactly one weight segment (every four steps issue one) behind it, 17
  // copies.  Copies retire in order, so every weight segment older than it
  // (among them the one step ks + 1 reads) has landed too; an activation
  // copy issued right after a weight segment is due four steps later.
  // Twelve steps (three segments) per loop trip, so that every stage and
  // buffer index is a constant: with ss = 3 q + sr, step ks = 4 ss + j has
  // stage (4 sr + j) % 6 and reads weight buffers sr and (sr + 1) % 3.
  auto step = [&](auto j_c, auto sr_c, int ss) {
    constexpr int j = decltype(j_c)::value;
    constexpr int sr = decltype(sr_c)::value;
    constexpr int sa = (4 * sr + j) % kSkAStages;                   // stage of step ks
    constexpr int sn = (sa + 1) % kSkAStages;                       // of step ks + 1
    constexpr int sp = (sa + kSkAStages - 1) % kSkAStages;          // of step ks - 1
    constexpr int wcur = sr, wnext = (sr + 1) % 3;
    const int ks = 4 * ss + j;
    issue_a(ks + 5 < last ? ks + 5 : last, sp);
    if constexpr (j == 3) issue_w(ss + 3 < nss - 1 ? ss + 3 : nss - 1, wcur);
    half8_t na[4], nb[4];
    Raw rn;
    read_a(IC<sn>{}, na);
    read_w(wbase + (j < 2 ? wcur : wnext) * kSkWStage, IC<(j + 2) & 3>{}, rn);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[jj], acc[i][jj], 0, 0, 0);
    dequant(rc, nb);
    // each product followed by one fragment read and a share of the
    // dequantisation
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tie_after(nb[i]);  // dequantised within this step, not sunk into the next
      fa[i] = na[i];
      fb[i] = nb[i];
    }
    rc = rn;
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<17>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compiler_fence();
  };
  auto segment = [&](auto sr_c, int ss) {
    step(IC<0>{}, sr_c, ss);
    step(IC<1>{}, sr_c, ss);
    step(IC<2>{}, sr_c, ss);
    step(IC<3>{}, sr_c, ss);
  };
  int ss = 0;
  for (; ss + 3 <= nss; ss += 3) {
    segment(IC<0>{}, ss);
    segment(IC<1>{}, ss + 1);
    segment(IC<2>{}, ss + 2);
  }
  if (ss < nss) segment(IC<0>{}, ss);
  if (ss + 1 < nss) segment(IC<1>{}, ss + 1);
  wait_vm_lgkm0<0>();
  __syncthreads();

  // Sum the four partial tiles, one 32-row fragment row at a time: each wave
  // writes its partial column-major (column stride kSkRedCol floats), then
  // thread t sums the 4 x 4 block of rows 4 (t % 8) .. + 3 and columns
  // 4 (t / 8) .. + 3 in wave order and stores each row's 4 columns with one
  // 8-byte (fp16) or 16-byte (fp32) store; a store instruction costs about
  // as much as a copy, so per-element stores made this epilogue several
  // microseconds long.
  float* red = reinterpret_cast<float*>(smem);
  const int rb4 = tid & 7, cb4 = tid >> 3;
  const int64_t col = n0 + 4 * cb4;
  const bool vec_ok = (ldy & 3) == 0 && col + 3 < n;
  bool bad = false;  // a non-finite sum (then the exact route rewrites the tile)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4_t v = {acc[i][jj][4 * q], acc[i][jj][4 * q + 1], acc[i][jj][4 * q + 2], acc[i][jj][4 * q + 3]};
        *reinterpret_cast<float4_t*>(red + (wave * 128 + 32 * jj + lc) * kSkRedCol + 8 * q + 4 * kg) = v;
      }
    __syncthreads();
    float4_t sc[4];  // column c of the block, rows 4 rb4 .. + 3
#pragma unroll
    for (int c = 0; c < 4; ++c) sc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sc[c] += *reinterpret_cast<const float4_t*>(red + (w * 128 + 4 * cb4 + c) * kSkRedCol + 4 * rb4);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) bad |= !__builtin_isfinite(sc[c][r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + 32 * i + 4 * rb4 + r;
      if (row >= m) continue;
      YT* dst = y + row * ldy + col;
      if (vec_ok) {
        if constexpr (sizeof(YT) == 2) {
          const half4_t h = {static_cast<half_t>(sc[0][r]), static_cast<half_t>(sc[1][r]),
                             static_cast<half_t>(sc[2][r]), static_cast<half_t>(sc[3][r])};
          *reinterpret_cast<half4_t*>(dst) = h;
        } else {
          *reinterpret_cast<float4_t*>(dst) = float4_t{sc[0][r], sc[1][r], sc[2][r], sc[3][r]};
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (col + c < n) dst[c] = static_cast<YT>(sc[c][r]);
      }
    }
    __syncthreads();
  }
  if (workgroup_any_flag(bad, reinterpret_cast<uint32_t*>(smem)))
    exact_tile128<256, YT>(xe, static_cast<DType>(xet), k, W0, rb, y, ldy, m, n, m0, n0,
                           2 * static_cast<int64_t>(ks0), 2 * static_cast<int64_t>(ks0 + nks),
                           reinterpret_cast<float*>(smem));
}

// Output columns c0 .. c0 + nc - 1 (weight rows c0 ..) into yc (their first
// column, row stride ldy); with splits > 1, split z of K goes to yc + z zstride.
// The original activations (the exact route's input): a pointer and dtype.
struct XSrc {
  const void* p;
  int dt;
};

template <int BM, int BN, int WVM, int WVN, typename YT>
hipError_t launch_tiled(const half_t* x, const uint8_t* packed, int64_t c0, int64_t nc, YT* yc,
                        int64_t m, int64_t k, int64_t ldy, int splits, int kps, int64_t zstride,
                        XSrc xe, hipStream_t s) {
  const uint8_t* w = packed + c0 * ((k / kQK) * kBlockBytes);
  void* argv[] = {const_cast<const half_t**>(&x), const_cast<const uint8_t**>(&w), &yc, &m,
                  &nc, &k, &ldy, &kps, &zstride, &xe.p, &xe.dt};
  const dim3 grid(static_cast<unsigned>((nc + BN - 1) / BN), static_cast<unsigned>((m + BM - 1) / BM),
                  static_cast<unsigned>(splits));
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_mfma_kernel<BM, BN, WVM, WVN, YT>),
                         grid, dim3(WVM * WVN * 64), argv, 0, s);
}

template <typename YT>
hipError_t launch_slicek(const half_t* x, const uint8_t* packed, int64_t c0, int64_t nc, YT* yc,
                         int64_t m, int64_t k, int64_t ldy, int splits, int kps, int64_t zstride,
                         XSrc xe, hipStream_t s) {
  const uint8_t* w = packed + c0 * ((k / kQK) * kBlockBytes);
  void* argv[] = {const_cast<const half_t**>(&x), const_cast<const uint8_t**>(&w), &yc, &m,
                  &nc, &k, &ldy, &kps, &zstride, &xe.p, &xe.dt};
  const dim3 grid(static_cast<unsigned>((nc + 127) / 128), static_cast<unsigned>((m + 127) / 128),
                  static_cast<unsigned>(splits));
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_slicek_kernel<YT>), grid, dim3(256),
                         argv, 0, s);
}

// y[r][c] = sum over z of part[z][r][c] (fixed order), 4 columns per thread.
template <typename YT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, YT* __restrict__ y,
                                                           int64_t m, int64_t nc, int64_t ldy, int splits) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // quad index
  const int64_t quads = m * nc / 4;
  if (q >= quads) return;
  const int64_t e = 4 * q, r = e / nc, c = e - r * nc;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) acc += *reinterpret_cast<const float4_t*>(part + z * m * nc + e);
#pragma unroll
  for (int i = 0; i < 4; ++i) y[r * ldy + c + i] = static_cast<YT>(acc[i]);
}

// Launch plan.  Columns [0, n_main) run `main` tiles over all of K in whole
// rounds of one tile per compute unit; columns [n_main, n) run `tail` tiles
// with K split `splits` ways (fp32 partials in the workspace, then one
// reduction in split order).  n_main = 0 splits every tile: a launch with
// fewer tiles than compute units (k/v projections of a 256-row chunk are 16
// slice-K tiles) then fills the chip with K splits instead of leaving most of
// it idle.  The candidates -- 256 x 256 or 128 x 128 main tiles, with or
// without a split tail, or every tile split -- are compared on a cost model
// whose constants were measured on MI355X (graph replays, one round of 256
// tiles, K from 1024 to 10240): a tile costs a fixed ~9.5 us (launch ramp,
// prologue copies, epilogue) plus per 64-wide k step ~2.05 us (256 x 256) or
// ~0.50 us (slice-K 128 x 128) with every compute unit busy, about a third
// less per step with few busy (the matrix cores are power-limited); a split
// adds its fp32 partial traffic and a reduction launch.
enum class Tile : int { Big = 0, SliceK = 1, Out128 = 2 };

struct GemmPlan {
  Tile main = Tile::Out128, tail = Tile::Out128;
  int64_t n_main = 0;
  int splits = 1, kps = 0;
  size_t ws_bytes = 0;
  double est_us = 0.0;
};

int tile_rows(Tile t) { return t == Tile::Big ? 256 : 128; }

// Estimated microseconds of one round of `wgs` workgroups of tile type t over
// `steps` 64-wide k steps on `cu` compute units.
double round_us(Tile t, int64_t steps, int64_t wgs, int64_t cu) {
  const double full = t == Tile::Big ? 2.05 : t == Tile::SliceK ? 0.50 : 0.86;
  const double fill = wgs >= cu ? 1.0 : static_cast<double>(wgs) / static_cast<double>(cu);
  return 9.5 + static_cast<double>(steps) * full * (0.65 + 0.35 * fill);
}

// Every tile of columns [c0, n) with K split s ways (s = 1: no split).
double split_us(Tile t, int64_t m, int64_t nc, int nks, int s, int kps, int64_t cu) {
  const int64_t bt = tile_rows(t);
  const int64_t tiles = ((m + bt - 1) / bt) * ((nc + bt - 1) / bt) * s;
  const int64_t rounds = (tiles + cu - 1) / cu;
  double us = 0.0;
  for (int64_t r = 0; r < rounds; ++r) {
    const int64_t w = r + 1 < rounds ? cu : tiles - r * cu;
    us += round_us(t, kps, w, cu);
  }
  if (s > 1) {
    const double part = static_cast<double>(s) * static_cast<double>(m * nc) * 4.0;
    us += 2.0 + 2.0 * part / 8.0e6;  // partials written, then read (mostly last-level cache)
  }
  (void)nks;
  return us;
}

// Steps per split for s splits of nks steps (whole 4-step segments for slice-K).
int split_kps(Tile t, int nks, int s) {
  int kps = (nks + s - 1) / s;
  if (t == Tile::SliceK) kps = (kps + 3) / 4 * 4;
  return kps;
}

GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k) {
  GemmPlan best;
  const int64_t cu = device_cu_count();
  const int nks = static_cast<int>(k / kBK);
  const bool sk_ok = k % 256 == 0 && k >= 1024;  // short k: prologue and reduction dominate
  const bool split_ok = k % kBK == 0 && n % 4 == 0;
  best.main = m >= 1024 ? Tile::Big : sk_ok ? Tile::SliceK : Tile::Out128;
  best.n_main = n;
  best.kps = nks;
  best.est_us = split_us(best.main, m, n, nks, 1, nks, cu);
  if (k % kBK != 0) return best;

  // 256 x 256 main tiles for m >= 1024 (128 x 128 slice-K tiles there only
  // when the 256 x 256 tiles would leave compute units idle: at full rounds
  // the 256 x 256 tile measured a few percent faster than the model says);
  // 128 x 128 tiles below, slice-K where k allows.
  const bool big_fills = ((m + 255) / 256) * ((n + 255) / 256) >= cu;
  std::initializer_list<Tile> mains = {Tile::Big, Tile::SliceK, Tile::Out128};
  for (Tile mt : mains) {
    if (mt == Tile::SliceK && (!sk_ok || (m >= 1024 && big_fills))) continue;
    if (mt == Tile::Out128 && (sk_ok || m >= 1024)) continue;  // slice-K is the faster 128 x 128 tile
    if (mt == Tile::Big && m < 1024) continue;
    const int64_t bt = tile_rows(mt);
    const int64_t tm = (m + bt - 1) / bt, tn = (n + bt - 1) / bt;
    auto consider = [&](const GemmPlan& c) {
      if (c.est_us < best.est_us) best = c;
    };
    // main tiles over every column, no split
    {
      GemmPlan c;
      c.main = c.tail = mt;
      c.n_main = n;
      c.kps = nks;
      c.est_us = split_us(mt, m, n, nks, 1, nks, cu);
      consider(c);
    }
    if (!split_ok) continue;
    // every tile split s ways
    if (tm * tn < cu) {
      for (int64_t s = 2; s <= cu / (tm * tn) && s <= nks; ++s) {
        GemmPlan c;
        c.main = c.tail = mt;
        c.n_main = 0;
        c.kps = split_kps(mt, nks, static_cast<int>(s));
        c.splits = (nks + c.kps - 1) / c.kps;
        if (c.splits < 2) continue;
        c.est_us = split_us(mt, m, n, nks, c.splits, c.kps, cu);
        c.ws_bytes = static_cast<size_t>(c.splits) * static_cast<size_t>(m * n) * 4;
        consider(c);
      }
    }
    // whole rounds of main tiles, the remaining columns split
    if (tm * tn > cu && (tm * tn) % cu != 0) {
      const int64_t tn_main = (tm * tn / cu) * cu / tm;
      if (tn_main >= 1 && tn_main < tn) {
        const int64_t nt = n - tn_main * bt;
        const double main_us = split_us(mt, m, tn_main * bt, nks, 1, nks, cu);
        for (Tile tt : mains) {
          if (tt == Tile::SliceK && !sk_ok) continue;
          if (tt == Tile::Out128 && sk_ok) continue;
          if (tt == Tile::Big && mt != Tile::Big) continue;
          const int64_t tb = tile_rows(tt);
          const int64_t ttiles = ((m + tb - 1) / tb) * ((nt + tb - 1) / tb);
          for (int64_t s = 2; s <= cu / ttiles && s <= nks; ++s) {
            GemmPlan c;
            c.main = mt;
            c.tail = tt;
            c.n_main = tn_main * bt;
            c.kps = split_kps(tt, nks, static_cast<int>(s));
            c.splits = (nks + c.kps - 1) / c.kps;
            if (c.splits < 2) continue;
            c.est_us = main_us + split_us(tt, m, nt, nks, c.splits, c.kps, cu);
            c.ws_bytes = static_cast<size_t>(c.splits) * static_cast<size_t>(m * nt) * 4;
            consider(c);
          }
        }
      }
    }
  }
  return best;
}

template <typename YT>
hipError_t launch_tile_type(Tile t, const half_t* x, const uint8_t* packed, int64_t c0, int64_t nc,
                            YT* yc, int64_t m, int64_t k, int64_t ldy, int splits, int kps,
                            int64_t zstride, XSrc xe, hipStream_t s) {
  if (t == Tile::Big)
    return launch_tiled<256, 256, 2, 4, YT>(x, packed, c0, nc, yc, m, k, ldy, splits, kps, zstride, xe, s);
  if (t == Tile::SliceK)
    return launch_slicek<YT>(x, packed, c0, nc, yc, m, k, ldy, splits, kps, zstride, xe, s);
  return launch_tiled<128, 128, 2, 2, YT>(x, packed, c0, nc, yc, m, k, ldy, splits, kps, zstride, xe, s);
}

template <typename YT>
hipError_t dispatch_tiled(const half_t* x, const uint8_t* packed, YT* y, int64_t m, int64_t n,
                          int64_t k, void* workspace, XSrc xe, hipStream_t s) {
  const GemmPlan p = gemm_plan(m, n, k);
  const int nks = static_cast<int>(k / kBK);
  hipError_t e = hipSuccess;
  if (p.n_main > 0) {
    e = launch_tile_type<YT>(p.main, x, packed, 0, p.n_main, y, m, k, n, 1, nks, 0, xe, s);
    if (e != hipSuccess || p.n_main == n) return e;
  }
  // Split columns: split z of K writes part[z], m x nt with row stride nt.
  const int64_t nt = n - p.n_main;
  float* part = static_cast<float*>(workspace);
  e = launch_tile_type<float>(p.tail, x, packed, p.n_main, nt, part, m, k, nt, p.splits, p.kps,
                              m * nt, xe, s);
  if (e != hipSuccess) return e;
  const int64_t quads = m * nt / 4;
  YT* yt = y + p.n_main;
  int sp = p.splits;
  int64_t ldy = n, mm = m, ntt = nt;
  void* argv[] = {&part, &yt, &mm, &ntt, &ldy, &sp};
  return hipLaunchKernel(reinterpret_cast<const void*>(&splitk_reduce_kernel<YT>),
                         dim3(static_cast<unsigned>((quads + 255) / 256)), dim3(256), argv, 0, s);
}

}  // namespace

namespace {

// Converted bf16 activations occupy the workspace's first bytes.
int64_t bf16_stage_bytes(int64_t m, int64_t k) { return (m * k * 2 + 255) / 256 * 256; }

// bf16 activations -> fp16 rows (round to nearest even), one workgroup of
// 256 threads per row (a 256-row chunk still fills the chip).  A row that
// holds any value fp16 cannot represent exactly (beyond its range, or off its
// subnormal grid) is written entirely as NaN instead: every tile and K split
// that reads it then ends with non-finite accumulators and is recomputed on
// the exact route from the bf16 original.  Both buffers are 16-byte aligned
// and k % 32 == 0.
__global__ __launch_bounds__(256) void bf16_rows_to_f16_kernel(const uint16_t* __restrict__ x,
                                                               uint16_t* __restrict__ out,
                                                               int64_t m, int64_t k) {
  const int64_t row = blockIdx.x;  // < m: one workgroup per row
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * k);
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * k);
  const int64_t np = k / 8;  // 16-byte pieces
  bool inexact = false;
  for (int64_t p = threadIdx.x; p < np; p += 256) {
    u32x4 v = src[p];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h = bf16x2_to_f16x2(v[e]);
      inexact |= !f16x2_holds_bf16x2(h, v[e]);
      v[e] = h;
    }
    dst[p] = v;
  }
  // (a separate kernel with no dynamic LDS: __syncthreads_or's own LDS is fine)
  if (__syncthreads_or(inexact)) {
    const u32x4 qnan = {0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u};
    for (int64_t p = threadIdx.x; p < np; p += 256) dst[p] = qnan;  // after this thread's own stores
  }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, DType xt) {
  if (xt == DType::F32) return 0;  // the exact route needs no workspace
  const size_t tiles = gemm_plan(m, n, k).ws_bytes;
  return xt == DType::BF16 ? static_cast<size_t>(bf16_stage_bytes(m, k)) + tiles : tiles;
}

hipError_t launch_gemm(const void* x, DType xt, const uint8_t* packed, void* y,
                       DType yt, int64_t m, int64_t n, int64_t k, void* workspace,
                       hipStream_t s) {
  const dim3 grid128(static_cast<unsigned>((n + 127) / 128), static_cast<unsigned>((m + 127) / 128));
  if (xt == DType::F32) {
    // fp32 activations: the exact route (fp32 matrix cores) for every tile.
    int xti = static_cast<int>(xt);
    void* argv[] = {const_cast<void**>(&x), &xti, const_cast<const uint8_t**>(&packed), &y,
                    &m, &n, &k};
    const void* fn = yt == DType::F16 ? reinterpret_cast<const void*>(&gemm_exact_kernel<half_t>)
                                      : reinterpret_cast<const void*>(&gemm_exact_kernel<float>);
    return hipLaunchKernel(fn, grid128, dim3(256), argv, 0, s);
  }
  const half_t* xp = static_cast<const half_t*>(x);
  const XSrc xe{x, static_cast<int>(xt)};
  if (xt == DType::BF16) {
    // Stage the activations as fp16 rows in the workspace (NaN rows where
    // fp16 cannot hold them exactly), then run the fp16 path on them with the
    // rest of the workspace; the exact route reads the bf16 original.
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const uint16_t* src = static_cast<const uint16_t*>(x);
    uint16_t* dst = reinterpret_cast<uint16_t*>(ws);
    int64_t mm = m, kk = k;
    void* argv[] = {&src, &dst, &mm, &kk};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bf16_rows_to_f16_kernel),
                                         dim3(static_cast<unsigned>(m)), dim3(256), argv, 0, s);
    if (e != hipSuccess) return e;
    xp = reinterpret_cast<const half_t*>(ws);
    workspace = gemm_plan(m, n, k).ws_bytes > 0 ? ws + bf16_stage_bytes(m, k) : nullptr;
  }
  if (k % kBK == 0) {
    if (yt == DType::F16)
      return dispatch_tiled(xp, packed, static_cast<half_t*>(y), m, n, k, workspace, xe, s);
    return dispatch_tiled(xp, packed, static_cast<float*>(y), m, n, k, workspace, xe, s);
  }
  const void* xev = xe.p;
  int xet = xe.dt;
  if (yt == DType::F16) {
    half_t* yp = static_cast<half_t*>(y);
    void* argv[] = {&xp, const_cast<const uint8_t**>(&packed), &yp, &m, &n, &k, &xev, &xet};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_tile_kernel<half_t>),
                           grid128, dim3(256), argv, 0, s);
  }
  float* yp = static_cast<float*>(y);
  void* argv[] = {&xp, const_cast<const uint8_t**>(&packed), &yp, &m, &n, &k, &xev, &xet};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_tile_kernel<float>),
                         grid128, dim3(256), argv, 0, s);
}

}  // namespace q4
