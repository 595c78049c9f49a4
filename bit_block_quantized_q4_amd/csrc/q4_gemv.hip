// Q4_0 batched-decode GEMV for gfx950: y[m][n] = x[m][k] . dequant(W)^T, m <= 32.
//
// The batched decode stage of the vertical-disaggregation page (section
// "Every cycle counts: custom kernels"): many sessions' decode steps share one
// pass over the weights, so each packed byte is read from HBM once for all m
// activation rows.  Every output is the fp32 sum over blocks of d times the
// exact block dot product of x with (q - 8); reductions run in a fixed order,
// so results are bit-reproducible.
//
// Streaming kernel (fp16 activations, k % 256 == 0)
// -------------------------------------------------
// A workgroup owns one 16-row tile of W; its NW wavefronts each take a
// contiguous share of K, cut into chunks of 8 blocks.  8 blocks are 144 bytes
// of a row, a multiple of 16, so a chunk of the tile is 144 coalesced 16-byte
// pieces.  Each wave streams its chunks through a private ring of R LDS slots
// with direct global->LDS copies (global_load_lds_dwordx4): the weight pieces
// and the chunk's activation rows travel together, so waiting for a slot is
// exactly "at most (R - 1) chunks of copies in flight" and never waits for a
// later copy (vector loads complete in order).  From the slot, per block, one
// v_mfma_f32_16x16x32_f16 (K = 32 is exactly one Q4_0 block):
//   A (16 x 32): activation rows m = lane % 16 (padding rows repeat row m-1);
//   B (32 x 16): the 16 weight rows, codes turned into exact fp16 (q - 8)
//                with byte permutes and the 1024+q / 64+q exponent trick;
//   D (16 x 16): lane l holds column l % 16, rows 4*(l/16) .. +3.
// Lane group g = l / 16 takes code bytes 4g..4g+3 of the block, i.e. elements
// 4g..4g+3 (low nibbles) and 4g+16..4g+19 (high nibbles); its A operand holds
// the activations of the same eight elements in the same order, so the
// contraction is the block dot product whatever k order the hardware uses.
// The block scale d (one per output column) is applied to the fresh block
// product with four fp32 FMAs.  The waves' partial tiles are summed in LDS in
// wave order at the end.
//
// Generic kernel (fp32 activations or k % 256 != 0): one wavefront per output
// feature, lanes stride over blocks, wave-wide xor-shuffle reduction.
#include "q4_device.hpp"

namespace q4 {
namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// ----------------------------------------------------------------- generic

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
hipError_t dispatch_rowwave(const void* x, const uint8_t* packed, void* y, int m,
                            int64_t n, int64_t k, hipStream_t s) {
  if (m <= 1) return launch_rowwave<XT, YT, 1>(x, packed, y, m, n, k, s);
  if (m <= 2) return launch_rowwave<XT, YT, 2>(x, packed, y, m, n, k, s);
  if (m <= 4) return launch_rowwave<XT, YT, 4>(x, packed, y, m, n, k, s);
  if (m <= 8) return launch_rowwave<XT, YT, 8>(x, packed, y, m, n, k, s);
  if (m <= 16) return launch_rowwave<XT, YT, 16>(x, packed, y, m, n, k, s);
  return launch_rowwave<XT, YT, 32>(x, packed, y, m, n, k, s);
}

// ----------------------------------------------------------------- streaming

constexpr int kTileRows = 16;                               // MFMA N
constexpr int kChunkBlocks = 8;                             // blocks per chunk
constexpr int kChunkRowBytes = kChunkBlocks * kBlockBytes;  // 144
constexpr int kChunkBytes = kTileRows * kChunkRowBytes;     // 2304
constexpr int kChunkPieces = kChunkBytes / 16;              // 144 x 16 B
constexpr int kPieceIters = (kChunkPieces + kWave - 1) / kWave;  // 3

// MT: 16-row m-tiles (1 or 2).  MX: activation rows staged per chunk (>= m,
// padding rows repeat row m - 1).  R: chunks in flight per wave.  NW: waves
// per workgroup, each taking a contiguous share of the tile's K chunks.
template <int MT, int MX, int R, int NW>
struct StreamCfg {
  static constexpr int kXRowPieces = 33;  // 32 pieces of a 512-byte row + 1 pad (bank spread)
  static constexpr int kXRowBytes = kXRowPieces * 16;
  static constexpr int kXBytes = MX * kXRowBytes;
  static constexpr int kSlot = kChunkBytes + kXBytes;
  static constexpr int kXPieces = MX * kXRowPieces;
  static constexpr int kXIters = (kXPieces + kWave - 1) / kWave;
  static constexpr int kXLast = kXPieces - kWave * (kXIters - 1);  // active lanes, last copy
  static constexpr int kOps = kPieceIters + kXIters;  // copies per chunk and lane
  static constexpr int kRed = NW * MT * 4 * kWave * 4;  // reduction scratch (aliases the ring)
  static constexpr int kLds = NW * R * kSlot > kRed ? NW * R * kSlot : kRed;
  static_assert((R - 1) * kOps < 64, "in-flight copies exceed the wait counter");
  static_assert(MX <= 16 * MT, "staged rows exceed the m-tiles");
};

template <int MT, int MX, int R, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_stream_kernel(
    const half_t* __restrict__ x, const uint8_t* __restrict__ W, void* __restrict__ y,
    int m, int64_t n, int64_t k, int y_f16) {
  using C = StreamCfg<MT, MX, R, NW>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::kLds];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nl = lane & 15;  // output column within the tile / A row
  const int g = lane >> 4;   // k group
  const int64_t rb = (k / kQK) * kBlockBytes;  // row bytes (multiple of 144)
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kTileRows;
  const int nchunks = static_cast<int>(k / (kQK * kChunkBlocks));
  const int c0 = (nchunks * wave) / NW;
  const int cpw = (nchunks * (wave + 1)) / NW - c0;  // this wave's chunks (may be 0)
  uint8_t* const ring = smem + wave * R * C::kSlot;

  // Weight pieces: copy q of a chunk moves piece p = lane + 64 q of the
  // 16 x 144-byte tile slice, row r = p / 9, 16-byte column j = p % 9, to
  // LDS byte 16 p (so LDS row r starts at 144 r).  Rows past n (a ragged last
  // tile) re-read row n - 1: their columns are never stored.
  const uint8_t* wsrc[kPieceIters];
#pragma unroll
  for (int q = 0; q < kPieceIters; ++q) {
    const int p = lane + kWave * q;
    const int r = p / 9;
    const int j = p - 9 * r;
    const int64_t row = row0 + r < n ? row0 + r : n - 1;
    wsrc[q] = W + row * rb + static_cast<int64_t>(c0) * kChunkRowBytes + 16 * (p < kChunkPieces ? j : 0);
  }
  // Activation pieces: LDS piece P = lane + 64 q holds row P / 33, 16-byte
  // column P % 33 of the chunk's 256 activations (column 32 is padding).
  // Rows past m repeat row m - 1.
  const half_t* xsrc[C::kXIters];
#pragma unroll
  for (int q = 0; q < C::kXIters; ++q) {
    const int P = lane + kWave * q;
    const int r = P / C::kXRowPieces;
    const int col = P - C::kXRowPieces * r;
    const int rr = r < m ? r : m - 1;
    xsrc[q] = x + static_cast<int64_t>(rr) * k + static_cast<int64_t>(c0) * kChunkBlocks * kQK +
              8 * (col < 32 ? col : 0);
  }
  auto issue = [&](int c, int s) {
    uint8_t* const sb = ring + s * C::kSlot;
#pragma unroll
    for (int q = 0; q < kPieceIters; ++q)
      if (q < kPieceIters - 1 || lane < kChunkPieces - kWave * (kPieceIters - 1))
        dma16(wsrc[q] + static_cast<int64_t>(c) * kChunkRowBytes, sb + kWave * 16 * q);
#pragma unroll
    for (int q = 0; q < C::kXIters; ++q)
      if (q < C::kXIters - 1 || lane < C::kXLast)
        dma16(xsrc[q] + static_cast<int64_t>(c) * kChunkBlocks * kQK,
              sb + kChunkBytes + kWave * 16 * q);
  };

  const UnpackConsts kc = make_unpack_consts();
  float4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Every iteration issues exactly one chunk's copies (past the end of the
  // wave's range the last chunk is re-read), so "chunk c has landed" is
  // always "at most (R - 1) chunks' copies still in flight".
  if (cpw > 0) {
#pragma unroll
    for (int s = 0; s < R; ++s) issue(s < cpw ? s : cpw - 1, s);
  }

  for (int c = 0; c < cpw; ++c) {
    const int s = c % R;
    wait_vm<(R - 1) * C::kOps>();
    const uint8_t* const sb = ring + s * C::kSlot;
    const uint8_t* const rowbase = sb + nl * kChunkRowBytes;
    const uint8_t* xrowp[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = 16 * t + nl;
      xrowp[t] = sb + kChunkBytes + (r < MX ? r : MX - 1) * C::kXRowBytes + 8 * g;
    }
    // Phase 1: every LDS read of the chunk, into distinct registers, so the
    // reads overlap each other instead of each block waiting for its own.
    uint32_t cw[kChunkBlocks][2];
    uint16_t dbits[kChunkBlocks];
    half8_t av[kChunkBlocks][MT];
#pragma unroll
    for (int j = 0; j < kChunkBlocks; ++j) {
      const uint8_t* blk = rowbase + j * kBlockBytes;
      dbits[j] = *reinterpret_cast<const uint16_t*>(blk);
      if ((j & 1) == 0) {  // codes start 2 bytes past a dword boundary
        const uint32_t* w = reinterpret_cast<const uint32_t*>(blk + 4 * g);
        cw[j][0] = w[0];
        cw[j][1] = w[1];
      } else {
        cw[j][0] = *reinterpret_cast<const uint32_t*>(blk + 2 + 4 * g);
        cw[j][1] = cw[j][0];
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint2 lo = *reinterpret_cast<const uint2*>(xrowp[t] + j * 64);
        const uint2 hi = *reinterpret_cast<const uint2*>(xrowp[t] + j * 64 + 32);
        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
        av[j][t] = __builtin_bit_cast(half8_t, a);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Phase 2: exact operands and independent block products.
    float4_t prod[kChunkBlocks][MT];
#pragma unroll
    for (int j = 0; j < kChunkBlocks; ++j) {
      const half8_t b = (j & 1) == 0 ? unpack8<2>(cw[j][0], cw[j][1], kc)
                                     : unpack8<0>(cw[j][0], cw[j][1], kc);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        prod[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[j][t], b,
                                                            float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Phase 3: scale application, in block order.
#pragma unroll
    for (int j = 0; j < kChunkBlocks; ++j) {
      const float d = half_bits_to_float(dbits[j]);
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = d * prod[j][t] + acc[t];
    }
    // The slot's LDS reads are consumed above; refill it with chunk c + R.
    compiler_fence();
    issue(c + R < cpw ? c + R : cpw - 1, s);
  }
  wait_vm<0>();

  // Fixed-order reduction of the waves' K shares (the ring is reused).
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [wave][t][i][lane]
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * MT + t) * 4 + i) * kWave + lane] = acc[t][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MT * 4 * kWave; idx += blockDim.x) {
    const int t = idx / (4 * kWave);
    const int i = (idx / kWave) % 4;
    const int l = idx % kWave;
    float sum = red[(t * 4 + i) * kWave + l];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[((w * MT + t) * 4 + i) * kWave + l];
    const int mm = 16 * t + 4 * (l >> 4) + i;
    const int64_t col = row0 + (l & 15);
    if (mm < m && col < n) {
      const int64_t o = static_cast<int64_t>(mm) * n + col;
      if (y_f16) static_cast<half_t*>(y)[o] = static_cast<half_t>(sum);
      else static_cast<float*>(y)[o] = sum;
    }
  }
}

template <int MT, int MX, int R, int NW>
hipError_t launch_stream(const void* x, const uint8_t* packed, void* y, bool y_f16, int m,
                         int64_t n, int64_t k, hipStream_t s) {
  static_assert(StreamCfg<MT, MX, R, NW>::kLds <= 160 * 1024, "LDS budget");
  const half_t* xp = static_cast<const half_t*>(x);
  int yf = y_f16 ? 1 : 0;
  void* argv[] = {&xp, const_cast<const uint8_t**>(&packed), &y, &m, &n, &k, &yf};
  const dim3 grid(static_cast<unsigned>((n + kTileRows - 1) / kTileRows));
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_stream_kernel<MT, MX, R, NW>), grid,
                         dim3(NW * kWave), argv, 0, s);
}

bool stream_supports(int64_t k) { return k % (kQK * kChunkBlocks) == 0; }

// Staged activation rows and waves per workgroup by batch size: the LDS ring
// (waves x 2 chunks x (2304 bytes of weights + 528 bytes per staged row))
// stays near 80 KB so two workgroups share a CU, except for m > 12.
hipError_t dispatch_stream(const void* x, const uint8_t* packed, void* y, bool y_f16, int m,
                           int64_t n, int64_t k, hipStream_t s) {
  if (m <= 1) return launch_stream<1, 1, 2, 10>(x, packed, y, y_f16, m, n, k, s);
  if (m <= 2) return launch_stream<1, 2, 2, 10>(x, packed, y, y_f16, m, n, k, s);
  if (m <= 4) return launch_stream<1, 4, 2, 8>(x, packed, y, y_f16, m, n, k, s);
  if (m <= 8) return launch_stream<1, 8, 2, 6>(x, packed, y, y_f16, m, n, k, s);
  if (m <= 12) return launch_stream<1, 12, 2, 4>(x, packed, y, y_f16, m, n, k, s);
  if (m <= 16) return launch_stream<1, 16, 2, 4>(x, packed, y, y_f16, m, n, k, s);
  return launch_stream<2, 32, 2, 4>(x, packed, y, y_f16, m, n, k, s);
}

}  // namespace

hipError_t launch_gemv(const void* x, DType xt, const uint8_t* packed, void* y,
                       DType yt, int m, int64_t n, int64_t k, hipStream_t s) {
  if (xt == DType::F16 && stream_supports(k))
    return dispatch_stream(x, packed, y, yt == DType::F16, m, n, k, s);
  if (xt == DType::F16) {
    if (yt == DType::F16) return dispatch_rowwave<half_t, half_t>(x, packed, y, m, n, k, s);
    return dispatch_rowwave<half_t, float>(x, packed, y, m, n, k, s);
  }
  if (yt == DType::F16) return dispatch_rowwave<float, half_t>(x, packed, y, m, n, k, s);
  return dispatch_rowwave<float, float>(x, packed, y, m, n, k, s);
}

}  // namespace q4
