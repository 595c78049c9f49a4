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
// Generic kernel (fp32 activations, or bf16 activations with k % 512 != 0,
// or k % 256 != 0): one wavefront per output feature, lanes stride over
// blocks, wave-wide xor-shuffle reduction.
//
// bf16 activations: the balanced and tile kernels convert them to fp16 in
// the kernel (round to nearest even; exact for every value fp16 represents)
// and then run their fp16 matrix-core path; the generic kernel widens them
// exactly to fp32.
#include "q4_device.hpp"

namespace q4 {
namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(bf16_t v) { return bf16_bits_to_float(v.bits); }

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

// ----------------------------------------------------------------- balanced

// Balanced kernel (fp16 activations, m <= 4, k % 512 == 0)
// ----------------------------------------------------------
// Rows are dealt out in groups of four, so every workgroup (one per compute
// unit) owns the same number of rows: 5120 rows are 20 per unit, 17408 are 68,
// 1024 are 4.  The products run on v_mfma_f32_4x4x4_16b_f16, sixteen
// independent 4 x 4 x 4 products per instruction:
//   lane l = 4 s + j holds slot s (operands A and B) and column j (B and D);
//   A_s (4 x 4): activation row i = l % 4 (rows past m repeat row m - 1);
//   B_s (4 x 4): weight row 4 rg + j, the same 4 elements, as exact (q - 8);
//   D_s (4 x 4): lane l, register i = activation row i, column j.
// Slot s is block s of a "set" of 16 consecutive blocks (512 values of k), so
// lane l owns one whole Q4_0 block of one weight row per task (a task is one
// row group of 4 rows times one set: 4 x 288 contiguous bytes).  Eight
// chained instructions walk the block's 32 elements: instruction (u, h) takes
// code bytes 4u .. 4u+3, low nibbles (elements 4u .. 4u+3) for h = 0 and high
// nibbles (elements 4u+16 .. 4u+19) for h = 1, so its A operand is two
// adjacent activation dwords.  The lane then scales the block product by its
// own block's d with one fp32 FMA per activation row.
//
// Data movement is all 16-byte direct global->LDS copies, coalesced: the
// workgroup first stages x (m rows of k halves), then each wave streams its
// tasks through a private LDS ring of P slots (72 pieces per task: the four
// 288-byte row segments).  Every task issues exactly two copies and the
// wave keeps at most P tasks in flight, so in steady state "task t has
// landed" is "at most 2 (P - 1) copies in flight"; the last P tasks wait for
// exact counts of the copies still behind them (no copies are wasted past the
// wave's last task).  Lanes read their block and
// activations from LDS.  Tasks are numbered row-group-major and dealt to the
// waves in contiguous ranges; a wave accumulates its current row group in
// registers and, when the row group changes, folds the 16 slots (two
// row-shift adds, then two cross-row shuffles) and stores one partial per
// weight row.  At the end every output sums the waves' partials in order.

constexpr int kSetBlocks = 16;
constexpr int kSetK = kSetBlocks * kQK;                   // 512
constexpr int kTaskRowBytes = kSetBlocks * kBlockBytes;   // 288 = 18 pieces
constexpr int kTaskBytes = 4 * kTaskRowBytes;             // 1152
constexpr int kTaskPieces = kTaskBytes / 16;              // 72

template <int V>
struct IC {
  static constexpr int value = V;
};

// LDS layout of a workgroup (byte offsets); shared by the kernel and the host.
struct BalLds {
  int64_t x_ops;   // 16-byte copies per wave for x
  int64_t x_bytes, ring_off, part_off, total;
};
__host__ __device__ inline BalLds bal_lds(int m, int64_t k, int rg, int nw, int p) {
  BalLds L;
  const int64_t pieces = (static_cast<int64_t>(m) * k * 2 + 15) / 16;
  L.x_ops = (pieces + nw * kWave - 1) / (nw * kWave);
  L.x_bytes = L.x_ops * nw * kWave * 16;
  L.ring_off = L.x_bytes;
  L.part_off = L.ring_off + static_cast<int64_t>(nw) * p * kTaskBytes;
  // [row group][wave][column j] float4 (zero where untouched)
  L.total = L.part_off + static_cast<int64_t>(rg) * nw * 4 * 16;
  return L;
}

// XB: the activations arrive as bf16 and are converted to fp16 in LDS, in
// place, once staged (exact for every value fp16 represents); if any
// conversion was not exact, the workgroup's rows are recomputed at the end on
// the exact route (gemv_exact_rows_bf16).
template <int NW, int P, int MR, bool XB>
__global__ __launch_bounds__(NW * kWave) void gemv_bal_kernel(
    const half_t* __restrict__ x, const uint8_t* __restrict__ W, void* __restrict__ y,
    int m, int64_t n, int64_t k, int rows_per_wg, int y_f16) {
  extern __shared__ __attribute__((aligned(16))) uint8_t bal_smem[];
  const int lane = threadIdx.x & (kWave - 1);
  // Wave-uniform (scalar) so that the task loop's control flow is uniform.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int nrows = static_cast<int>(n - r0 < rows_per_wg ? n - r0 : rows_per_wg);
  const int RG = (nrows + 3) >> 2;
  const int S = static_cast<int>(k / kSetK);
  const int T = RG * S;
  const int t0 = static_cast<int>((static_cast<int64_t>(T) * wave) / NW);
  const int t1 = static_cast<int>((static_cast<int64_t>(T) * (wave + 1)) / NW);
  const int64_t rb = (k / kQK) * kBlockBytes;
  const BalLds L = bal_lds(m, k, RG, NW, P);
  uint8_t* const xs = bal_smem;
  uint8_t* const ring = bal_smem + L.ring_off + static_cast<int64_t>(wave) * P * kTaskBytes;
  float4_t* const part = reinterpret_cast<float4_t*>(bal_smem + L.part_off);
  for (int i = threadIdx.x; i < RG * NW * 4; i += NW * kWave) part[i] = float4_t{0.f, 0.f, 0.f, 0.f};

  // x staging: wave w copies pieces (w * x_ops + q) * 64 + lane; pieces past
  // the end re-read the last piece into the padding of the region.
  {
    const int64_t pieces = (static_cast<int64_t>(m) * k * 2 + 15) / 16;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
    for (int64_t q = 0; q < L.x_ops; ++q) {
      const int64_t blk = static_cast<int64_t>(wave) * L.x_ops + q;
      int64_t pc = blk * kWave + lane;
      if (pc > pieces - 1) pc = pieces - 1;
      dma16(xb + 16 * pc, xs + blk * kWave * 16);
    }
  }

  // Task copies: piece p = lane (first copy) and 64 + lane (second copy,
  // lanes 0..7) of the 4 x 18 pieces; piece p is row p / 18, column p % 18.
  const int pj0 = lane / 18, pc0 = lane - 18 * (lane / 18);
  const int pj1 = (kWave + lane) / 18, pc1 = (kWave + lane) - 18 * ((kWave + lane) / 18);
  // Sources of the lane's two pieces in set 0 of row group rg (rows past n
  // re-read row n - 1: a ragged last group is computed, never stored).
  const uint8_t* src0 = W;
  const uint8_t* src1 = W;
  auto set_rows = [&](int rg) {
    int64_t row0 = r0 + 4 * rg + pj0, row1 = r0 + 4 * rg + pj1;
    if (row0 > n - 1) row0 = n - 1;
    if (row1 > n - 1) row1 = n - 1;
    src0 = W + row0 * rb + 16 * pc0;
    src1 = W + row1 * rb + 16 * pc1;
  };
  // Non-temporal copies: every packed byte is read once (34816 x 5120 m = 1:
  // 22.4 -> 21.1 us; 5120 x 17408: 12.5 -> 11.6 us; bit-identical).
  auto issue_task = [&](int st, int slot) {
    uint8_t* dst = ring + slot * kTaskBytes;
    const int64_t base = static_cast<int64_t>(st) * kTaskRowBytes;
    dma16_nt(src0 + base, dst);
    if (lane < kTaskPieces - kWave) dma16_nt(src1 + base, dst + kWave * 16);
  };

  const int j = lane & 3;    // B/D column: weight row within the group; A row
  const int sl = lane >> 2;  // slot: block within the set
  const bool odd = (sl & 1) != 0;  // block parity (sets start on even blocks)
  // Byte selectors on the window {w[u+1]:w[u]} of the lane's five dwords:
  // code bytes 4u, 4u+1 (sel_a) and 4u+2, 4u+3 (sel_b) as [c, 0, c', 0]; code
  // byte b sits at window offset b + 2 in an even block and b in an odd one.
  // dsel picks the scale's two bytes.
  const uint32_t sel_a = odd ? 0x0c010c00u : 0x0c030c02u;
  const uint32_t sel_b = odd ? 0x0c030c02u : 0x0c050c04u;
  const uint32_t dsel = odd ? 0x0c0c0706u : 0x0c0c0100u;
  // The lane's five dwords in the slot: [w0..w3] from the block start (even
  // block) or start + 2 (odd), and w4 at start + 16 (even) or start - 2 (odd);
  // all inside the slot's row segment.
  const int blk_off = kTaskRowBytes * j + kBlockBytes * sl;
  const int off4 = blk_off + (odd ? 2 : 0);
  const int off1 = blk_off + (odd ? -2 : 16);
  const int mm = j < m ? j : m - 1;
  const UnpackConsts kc = make_unpack_consts();
  const half2_t klo = {static_cast<half_t>(-1032.0f), static_cast<half_t>(-1032.0f)};
  const half2_t khi = {static_cast<half_t>(-72.0f), static_cast<half_t>(-72.0f)};

  float4_t accr = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint8_t* slot, int st) {
    const uint32_t* wv = reinterpret_cast<const uint32_t*>(slot + off4);
    const uint32_t w0 = wv[0], w1 = wv[1], w2 = wv[2], w3 = wv[3];
    const uint32_t w4 = *reinterpret_cast<const uint32_t*>(slot + off1);
    const u32x4* xa = reinterpret_cast<const u32x4*>(
        xs + (static_cast<int64_t>(mm) * k + static_cast<int64_t>(kSetBlocks * st + sl) * kQK) * 2);
    const u32x4 xr[4] = {xa[0], xa[1], xa[2], xa[3]};
    const float d = half_bits_to_float(static_cast<uint16_t>(__builtin_amdgcn_perm(w4, w0, dsel)));
    float4_t D;
    // A operand of (u, h): activation dwords 8h + 2u and 8h + 2u + 1.
    auto a_op = [&](auto uu, auto hh) {
      constexpr int dw = 8 * decltype(hh)::value + 2 * decltype(uu)::value;
      const u32x2 pr = {xr[dw >> 2][dw & 3], xr[dw >> 2][(dw & 3) + 1]};
      return __builtin_bit_cast(half4_t, pr);
    };
    // Code dword u is the byte window {hi:lo} = {w[u + 1] : w[u]}.
    auto dword = [&](auto uu, uint32_t hi, uint32_t lo) {
      constexpr int u = decltype(uu)::value;
      const uint32_t t01 = __builtin_amdgcn_perm(hi, lo, sel_a);
      const uint32_t t23 = __builtin_amdgcn_perm(hi, lo, sel_b);
      const half2_t l01 = __builtin_bit_cast(half2_t, (t01 & kc.mask_lo) | kc.exp_lo) + klo;
      const half2_t l23 = __builtin_bit_cast(half2_t, (t23 & kc.mask_lo) | kc.exp_lo) + klo;
      const half2_t h01 = __builtin_bit_cast(half2_t, (t01 & kc.mask_hi) | kc.exp_hi) + khi;
      const half2_t h23 = __builtin_bit_cast(half2_t, (t23 & kc.mask_hi) | kc.exp_hi) + khi;
      const half4_t Blo = {l01[0], l01[1], l23[0], l23[1]};
      const half4_t Bhi = {h01[0], h01[1], h23[0], h23[1]};
      D = __builtin_amdgcn_mfma_f32_4x4x4f16(a_op(uu, IC<0>{}), Blo,
                                             u == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : D, 0, 0, 0);
      D = __builtin_amdgcn_mfma_f32_4x4x4f16(a_op(uu, IC<1>{}), Bhi, D, 0, 0, 0);
    };
    dword(IC<0>{}, w1, w0);
    dword(IC<1>{}, w2, w1);
    dword(IC<2>{}, w3, w2);
    dword(IC<3>{}, w4, w3);
#pragma unroll
    for (int i = 0; i < MR; ++i) accr[i] = d * D[i] + accr[i];
  };

  // Fold of the 16 slots per row of 16 lanes: after two row-shift adds lane
  // 16 R + 12 + j holds the sum over slots 4R .. 4R+3 for weight row j.
  // (The element is copied to a scalar before the bit cast: a bit cast of a
  // vector element expression has been compiled as a read of element 0.)
  auto dpp_add = [](float4_t v, auto ctrl) {
    constexpr int c = decltype(ctrl)::value;
    float4_t r = v;
#pragma unroll
    for (int e = 0; e < MR; ++e) {
      const float ve = v[e];
      const int sh = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, ve), c, 0xF, 0xF, true);
      r[e] = ve + __builtin_bit_cast(float, sh);
    }
    return r;
  };
  auto flush = [&](int rg) {
    float4_t v = dpp_add(accr, IC<0x118>{});  // row_shr:8
    v = dpp_add(v, IC<0x114>{});               // row_shr:4
    // ... then the four rows of lanes: (R0 + R1) + (R2 + R3) into row 0.
#pragma unroll
    for (int e = 0; e < MR; ++e) {
      const float ve = v[e];
      const float a = ve + __shfl_xor(ve, 16);
      v[e] = a + __shfl_xor(a, 32);
    }
    if (lane >= 12 && lane < 16) part[(rg * NW + wave) * 4 + (lane & 3)] = v;
    accr = float4_t{0.f, 0.f, 0.f, 0.f};
  };

  // bf16 activations: every wave's x copies have landed (the barrier before
  // this); convert the staged rows to fp16 in place, then a second barrier
  // (task copies stay in flight through it).
  bool inexact = false;  // a bf16 activation that fp16 does not hold exactly
  auto convert_x = [&]() {
    if constexpr (XB) {
      // 16-byte pieces (eight values), four per thread in flight
      u32x4* xq = reinterpret_cast<u32x4*>(xs);
      const int64_t nq = static_cast<int64_t>(m) * k / 8;
      constexpr int kT = NW * kWave;
      int64_t i = threadIdx.x;
      for (; i + 3 * kT < nq; i += 4 * kT) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = xq[i + u * kT];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t h = bf16x2_to_f16x2(v[u][e]);
            inexact |= !f16x2_holds_bf16x2(h, v[u][e]);
            v[u][e] = h;
          }
          xq[i + u * kT] = v[u];
        }
      }
      for (; i < nq; i += kT) {
        u32x4 v = xq[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h = bf16x2_to_f16x2(v[e]);
          inexact |= !f16x2_holds_bf16x2(h, v[e]);
          v[e] = h;
        }
        xq[i] = v;
      }
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
    }
  };

  static_assert((P & (P - 1)) == 0, "ring size must be a power of two");
  if (t0 < t1) {
    const int ntask = t1 - t0;
    int lrg = t0 / S, lset = t0 - (t0 / S) * S, issued = 0;
    set_rows(lrg);
    auto next_copy = [&]() {  // task `issued` of this wave into slot issued % P
      issue_task(lset, issued & (P - 1));
      ++issued;
      if (++lset == S) {
        lset = 0;
        set_rows(++lrg);
      }
    };
    const int npro = ntask < P ? ntask : P;
    for (int i = 0; i < npro; ++i) next_copy();
    // This wave's x copies (issued before its 2 npro task copies) and its
    // partial-sum zeroing are complete; the barrier extends that to every wave.
    wait_vm_lgkm0_upto<2 * P>(2 * npro);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    convert_x();
    int cset = t0 - (t0 / S) * S, crg = t0 / S;
    auto finish = [&](int t) {
      compute(ring + (t & (P - 1)) * kTaskBytes, cset);
      if (++cset == S) {  // row group complete
        cset = 0;
        flush(crg);
        ++crg;
      }
    };
    // Steady state: task t has landed when at most 2 (P - 1) copies are in
    // flight; its slot is then refilled with task t + P.
    int t = 0;
    for (; t + P < ntask; ++t) {
      wait_vm<2 * (P - 1)>();
      compiler_fence();
      finish(t);
      compiler_fence();  // the slot's reads are consumed above
      next_copy();
    }
    // The last r <= P tasks are all in flight; nothing more is copied.
    const int r = ntask - t;
    for (int q = 0; q < r; ++q) {
      wait_vm_upto<2 * (P - 1)>(2 * (r - 1 - q));
      compiler_fence();
      finish(t + q);
    }
    if (cset != 0) flush(crg);  // the last row group was only partly this wave's
  } else {
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();  // matches the barrier of the waves with tasks
    convert_x();
  }

  __syncthreads();
  const int O = nrows * m;
  const float* pf = reinterpret_cast<const float*>(part);
  for (int o = threadIdx.x; o < O; o += NW * kWave) {
    const int rl = o / m, mo = o - (o / m) * m;
    const int rg = rl >> 2, jj = rl & 3;
    const float* q = pf + static_cast<int64_t>(rg) * NW * 16 + jj * 4 + mo;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += q[w * 16];
    const int64_t off = static_cast<int64_t>(mo) * n + r0 + rl;
    if (y_f16) static_cast<half_t*>(y)[off] = static_cast<half_t>(sum);
    else static_cast<float*>(y)[off] = sum;
  }
  if constexpr (XB) {
    if (workgroup_any_flag(inexact, reinterpret_cast<uint32_t*>(bal_smem)))
      gemv_exact_rows_bf16<NW>(reinterpret_cast<const uint16_t*>(x), W, y, y_f16, m, n, k, r0, nrows);
  }
}

constexpr int64_t kLdsMax = 160 * 1024;
constexpr int kBalP = 4;  // tasks in flight per wave
// Two tasks in flight per wave where four do not leave room in LDS for the
// staged activations (m = 4 at k = 17408: 139 KB of x), for workgroups of at
// most 32 rows: measured 16.4 -> 14.8 us at 5120 x 17408, m = 4 (against the
// tile kernel), but 32.7 -> 38.8 us at 16384 x 16384 (64 rows per workgroup,
// too little in flight for that much work), which keeps the tile kernel.
constexpr int kBalPSmall = 2;
constexpr int kBalPSmallMaxGroups = 8;


struct BalPlan {
  int rows_per_wg = 0, grid = 0, nw = 0, ring = 0;
  int64_t lds = 0;
};

// Rows per workgroup: a multiple of 4 near n / (compute units).  Returns false
// when the shape is outside the kernel (the caller uses the other kernels).
bool bal_plan(int m, int64_t n, int64_t k, BalPlan* p) {
  if (m < 1 || m > 4 || k % kSetK != 0) return false;
  const int64_t cu = device_cu_count();
  const int64_t rows = 4 * ((n + 4 * cu - 1) / (4 * cu));
  if (rows > (1 << 20)) return false;
  p->rows_per_wg = static_cast<int>(rows);
  p->grid = static_cast<int>((n + rows - 1) / rows);
  const int rg = static_cast<int>(rows / 4);
  const int tries[3][2] = {{8, kBalP}, {16, kBalP}, {8, kBalPSmall}};  // {waves, ring}
  for (const auto& t : tries) {
    if (t[1] == kBalPSmall && rg > kBalPSmallMaxGroups) break;
    const BalLds L = bal_lds(m, k, rg, t[0], t[1]);
    if (L.total <= kLdsMax) {
      p->nw = t[0];
      p->ring = t[1];
      p->lds = L.total;
      return true;
    }
  }
  return false;
}

template <int NW, int P, int MR, bool XB>
hipError_t launch_bal_t(const void* x, const uint8_t* packed, void* y, bool y_f16, int m,
                        int64_t n, int64_t k, const BalPlan& p, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&gemv_bal_kernel<NW, P, MR, XB>);
  static std::atomic<uint64_t> lds_allowed{0};
  const hipError_t e = allow_dynamic_lds(fn, static_cast<int>(kLdsMax), lds_allowed);
  if (e != hipSuccess) return e;
  const half_t* xp = static_cast<const half_t*>(x);
  int rows = p.rows_per_wg, yf = y_f16 ? 1 : 0;
  void* argv[] = {&xp, const_cast<const uint8_t**>(&packed), &y, &m, &n, &k, &rows, &yf};
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(p.grid)), dim3(NW * kWave), argv,
                         static_cast<size_t>(p.lds), s);
}

template <int MR, bool XB>
hipError_t dispatch_bal_m(const void* x, const uint8_t* packed, void* y, bool y_f16, int m,
                          int64_t n, int64_t k, const BalPlan& p, hipStream_t s) {
  if (p.ring == kBalPSmall) return launch_bal_t<8, kBalPSmall, MR, XB>(x, packed, y, y_f16, m, n, k, p, s);
  if (p.nw == 16) return launch_bal_t<16, kBalP, MR, XB>(x, packed, y, y_f16, m, n, k, p, s);
  return launch_bal_t<8, kBalP, MR, XB>(x, packed, y, y_f16, m, n, k, p, s);
}

// MR: activation rows accumulated (m rounded up to 1, 2 or 4).
template <bool XB>
hipError_t dispatch_bal(const void* x, const uint8_t* packed, void* y, bool y_f16, int m,
                        int64_t n, int64_t k, const BalPlan& p, hipStream_t s) {
  if (m == 1) return dispatch_bal_m<1, XB>(x, packed, y, y_f16, m, n, k, p, s);
  if (m == 2) return dispatch_bal_m<2, XB>(x, packed, y, y_f16, m, n, k, p, s);
  return dispatch_bal_m<4, XB>(x, packed, y, y_f16, m, n, k, p, s);
}

}  // namespace

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

hipError_t launch_gemv(const void* x, DType xt, const uint8_t* packed, void* y,
                       DType yt, int m, int64_t n, int64_t k, hipStream_t s) {
  BalPlan plan;
  const bool xh = xt == DType::F16, xb = xt == DType::BF16;
  if (xh && bal_plan(m, n, k, &plan))
    return dispatch_bal<false>(x, packed, y, yt == DType::F16, m, n, k, plan, s);
  if (xb && bal_plan(m, n, k, &plan))
    return dispatch_bal<true>(x, packed, y, yt == DType::F16, m, n, k, plan, s);
  if ((xh || xb) && gemv_tile_supports(m, k))
    return launch_gemv_tile(x, xb, packed, y, yt == DType::F16, m, n, k, s);
  if (xh && stream_supports(k))
    return dispatch_stream(x, packed, y, yt == DType::F16, m, n, k, s);
  if (xh) {
    if (yt == DType::F16) return dispatch_rowwave<half_t, half_t>(x, packed, y, m, n, k, s);
    return dispatch_rowwave<half_t, float>(x, packed, y, m, n, k, s);
  }
  if (xb) {
    if (yt == DType::F16) return dispatch_rowwave<bf16_t, half_t>(x, packed, y, m, n, k, s);
    return dispatch_rowwave<bf16_t, float>(x, packed, y, m, n, k, s);
  }
  if (yt == DType::F16) return dispatch_rowwave<float, half_t>(x, packed, y, m, n, k, s);
  return dispatch_rowwave<float, float>(x, packed, y, m, n, k, s);
}

}  // namespace q4
