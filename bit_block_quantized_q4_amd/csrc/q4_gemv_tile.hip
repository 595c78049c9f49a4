// Q4_0 decode GEMV on 16 x 16 x 32 matrix cores: y[i, r] = sum_j x[i, j] w[r, j]
// for a batch of up to 32 activation rows (the batched decode stage of
// "Vertical disaggregation: maximizing throughput on heterogeneous silicon",
// section "Every cycle counts: custom kernels", over its one shared Q4_0
// weight format).
//
// One workgroup owns R <= 16 T consecutive weight rows over the whole of K,
// so no partial sums leave the workgroup.  When R is not a multiple of 16
// (rows spread over every compute unit) the last row tile is partial: its
// unfilled rows hold stale bytes, feed only their own outputs and are never
// stored.  K is walked in phases of PB blocks (32 PB weights).  For every
// phase NP copying waves (four; two where two workgroups share a compute
// unit) copy, global -> LDS, the phase's weight bytes of the R rows and the
// phase's activation columns (16-byte copies); three phases are resident in
// a ring, so the copies of phases p + 1 and p + 2 are in flight while NW
// computing waves (eight, or four) work on phase p.  Within a phase wave w
// owns blocks w PB / NW .. (w + 1) PB / NW - 1 for all 16 T rows;
// each (row tile, block) pair is one v_mfma_f32_16x16x32_f16 with 16
// activation rows on the A side and 16 weight rows on the B side.  The
// block's 32 codes enter as exact fp16 integers q - 8 (the 1024 + q / 64 + q
// exponent trick and one exact packed subtraction), so every product x (q - 8)
// is exact and the block sum's rounding error is relative to
// sum |x (q - 8)|; the block scale d is then applied in fp32 to the 4
// outputs the lane holds (lane l: weight row l % 16, activation rows
// 4 (l / 16) .. +3).  (An earlier form fed the codes as fp16 subnormals
// q 2^-24 and carried -8 2^-24 sum(x) through a separately rounded
// accumulator input; its error then scaled with sum |x| instead of
// sum |x w| and could exceed the tolerance on blocks where large activations
// meet zero weights.)
//
// Bank layout: a weight row occupies an odd number of 16-byte pieces (the
// phase's 9 PB / 8 data pieces plus one padding piece), so the 16 rows one
// column read touches fall in 8 distinct bank quads (2-way at most); an
// activation row's 16-byte pieces are stored XOR-swizzled by the row index,
// so the 16 rows one operand read touches spread over all banks.
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int kTLdsMax = 160 * 1024;

#ifdef Q4_PHASE_TRACE
// Measurement build only (libq4trace.so, never libq4.so): each computing wave
// records the shader clock (s_memtime) at entry (slot 0), after phase p's
// barrier (1 + p) and after phase p's products (32 + p), p < 30, and at the
// end (63), and the constant 100 MHz clock (s_memrealtime) at entry (31) and
// at the end (62), so that the shader clock's rate over the launch is known,
// into a buffer the caller sets with q4_phase_trace_set:
// [workgroup][computing wave][64] uint64.
__device__ uint64_t* g_phase_trace = nullptr;
// The buffer's address is read once, at entry (a store through it could
// otherwise alias the variable and force a reload at every mark).
#define Q4_PHASE_TRACE_BEGIN \
  uint64_t* const phase_trace_ = wave < NW ? g_phase_trace : nullptr;
#define Q4_PHASE_STAMP(ev, clock)                                                     \
  do {                                                                                \
    if (phase_trace_ != nullptr) {                                                    \
      const uint64_t t_ = clock();                                                    \
      if (lane == 0)                                                                  \
        phase_trace_[(static_cast<int64_t>(blockIdx.x) * NW + wave) * 64 + (ev)] = t_; \
    }                                                                                 \
  } while (0)
#define Q4_PHASE_MARK(ev) Q4_PHASE_STAMP(ev, __builtin_amdgcn_s_memtime)
#define Q4_PHASE_MARK_RT(ev) Q4_PHASE_STAMP(ev, __builtin_amdgcn_s_memrealtime)
#else
#define Q4_PHASE_TRACE_BEGIN
#define Q4_PHASE_MARK(ev) \
  do {                    \
  } while (0)
#define Q4_PHASE_MARK_RT(ev) \
  do {                       \
  } while (0)
#endif
// Row tiles from which the end-of-launch sum takes a lane's whole fragment
// per thread (see the kernel's last step).
constexpr int kTileFragSum = 5;
// Phases resident in LDS.  (Deeper rings of smaller phases, 16 blocks in up
// to seven slots, measured slower than three slots of 32 blocks at
// 5120 x 5120: the per-phase barrier and fixed costs outweigh the extra
// copies in flight.)
constexpr int kTSlots = 3;

template <int V>
struct TC {
  static constexpr int value = V;
};

// Unrolled loop over a compile-time range: f(TC<0>{}), ..., f(TC<N - 1>{}).
template <int I, int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (I < N) {
    f(TC<I>{});
    unroll<I + 1, N>(f);
  }
}

// Geometry of one phase slot for T row tiles, AT activation tiles, PB blocks
// per phase, NW computing waves and NP copying waves (NP = 0: the computing
// waves copy too).  WR (<= 16 T) is the weight rows a slot holds: below 16 T
// the last tile's rows past WR read bytes of the slot's activation area
// (in bounds; they feed only outputs that are never stored), which lets
// three slots of 5 tiles x 2 activation tiles fit the LDS.  XR (<= 16 AT)
// is the activation rows a slot holds: a launch needs m <= XR, and operand
// rows past m read row m - 1, so a smaller area (nine tiles with m <= 10)
// leaves the LDS to weight rows.
template <int T, int AT, int PB, int NW, int NP, int WR = 16 * T, int XR = 16 * AT>
struct TileGeo {
  static constexpr int nw = NW;
  static constexpr int lanes = (NW + NP) * kWave;         // threads of the workgroup
  static constexpr int cwaves = NP > 0 ? NP : NW;         // copying waves
  static constexpr int clanes = cwaves * kWave;
  static constexpr int jb = PB / NW;                      // blocks per wave per phase
  static constexpr int row_pc = PB * kBlockBytes / 16;    // weight pieces per row
  static constexpr int wstride_pc = row_pc + 1;           // odd row stride (pieces)
  static constexpr int wstride = 16 * wstride_pc;
  static_assert(WR >= 1 && WR <= 16 * T, "weight rows of a slot");
  static constexpr int wpos = WR * wstride_pc;             // weight pieces per slot
  static constexpr int niw = (wpos + clanes - 1) / clanes;  // copy rounds (max per wave)
  static constexpr int wbytes = (16 * wpos + 255) / 256 * 256;
  static constexpr int xp = PB * kQK * 2 / 16;            // 16-byte pieces per activation row
  static_assert(XR >= 1 && XR <= 16 * AT, "activation rows of a slot");
  static constexpr int nix_max = (XR * xp + clanes - 1) / clanes;
  static constexpr int xbytes = XR * xp * 16;
  static constexpr int slot = wbytes + xbytes;
  static constexpr int red = T * AT * NW * kWave * 16;
  static constexpr int lds = kTSlots * slot > red ? kTSlots * slot : red;
  static constexpr int phase_k = PB * kQK;
  static constexpr int ndma = niw + nix_max;              // copy instructions per phase (max)
  static constexpr int tiles = T * jb;                    // (row tile, block) pairs per wave
  static constexpr int dma_per_tile = (ndma + tiles - 1) / tiles;
  static_assert(PB % (2 * NW) == 0, "blocks per wave must be even");
  static_assert((PB * kBlockBytes) % 16 == 0, "row segments of whole pieces");
  static_assert(xp >= 16, "swizzle needs 16 pieces per row");
};

// FULL: every workgroup owns 16 T rows (the last one's rows past n copy row
// n - 1 and are not stored); otherwise R = rows < 16 T rows and only those
// are copied (a run-time bound on the copies).  XB: the activations are bf16;
// each operand fragment is converted to fp16 in registers after its LDS read
// (round to nearest even, exact for every value fp16 represents) and checked
// to be exact; if any conversion of the workgroup was not, its rows are
// recomputed on the exact route (gemv_exact_rows_bf16).  (Having
// the copying waves convert their own pieces in LDS before the phase barrier
// instead measured slower: 12.3 against 8.9 us at 5120 x 5120, m = 16, as it
// delays the barrier and the next phase's copies.)
template <int T, int AT, int PB, bool FULL, int NW, int NP, bool XB, int WR, int XR>
__global__ __launch_bounds__((NW + NP) * kWave, 1) void gemv_tile_kernel(
    const half_t* __restrict__ x, const uint8_t* __restrict__ W, void* __restrict__ y, int m,
    int64_t n, int64_t k, int y_f16, int rows) {
  using G = TileGeo<T, AT, PB, NW, NP, WR, XR>;
  static_assert(!FULL || WR == 16 * T, "a full workgroup copies 16 T rows");
  constexpr int CW = G::cwaves;
  extern __shared__ __attribute__((aligned(16))) uint8_t tsm[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // copying-wave index (waves NW .. NW + NP - 1 copy when NP > 0)
  const int cwave = NP > 0 ? (wave >= NW ? wave - NW : 0) : wave;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * rows;
  const int rv = static_cast<int>(n - row0 < rows ? n - row0 : rows);  // rows stored
  const int64_t rb = (k / kQK) * kBlockBytes;  // bytes per weight row
  const int nph = static_cast<int>(k / G::phase_k);
  const uint32_t smem = lds_addr(tsm);
  Q4_PHASE_TRACE_BEGIN
  Q4_PHASE_MARK(0);
  Q4_PHASE_MARK_RT(31);

  // Weight copies.  Slot piece i = (q CW + cwave) 64 + lane holds piece
  // i % wstride_pc of the phase's segment of row i / wstride_pc (the padding
  // piece repeats the last one).  FULL: all 16 T rows are copied (rows past
  // n read row n - 1); otherwise only the rv rows of the workgroup.  Lanes
  // past the copied pieces copy nothing, and a wave issues the rounds q in
  // which any of its lanes copies (cw of them).
  const int wpos = FULL ? G::wpos : rv * G::wstride_pc;
  uint32_t wsrc[G::niw];
#pragma unroll
  for (int q = 0; q < G::niw; ++q) {
    int i = (q * CW + cwave) * kWave + lane;
    if (i > wpos - 1) i = wpos - 1;
    const int r = i / G::wstride_pc;
    int c = i - r * G::wstride_pc;
    if (c > G::row_pc - 1) c = G::row_pc - 1;
    int64_t grow = row0 + r;
    if (grow > n - 1) grow = n - 1;
    wsrc[q] = static_cast<uint32_t>((grow - row0) * rb + 16 * c);
  }
  int cw = 0;
#pragma unroll
  for (int q = 0; q < G::niw; ++q) cw += ((q * CW + cwave) * kWave < wpos) ? 1 : 0;
  // Activation copies: piece position i of the slot's activation area holds
  // piece (i % xp) ^ (row & 15) of row i / xp of the phase's columns; only
  // the m real rows are copied (a wave issues the cx rounds in which any of
  // its lanes copies).
  const int xpos = m * G::xp;
  int cx = 0;
#pragma unroll
  for (int q = 0; q < G::nix_max; ++q) cx += ((q * CW + cwave) * kWave < xpos) ? 1 : 0;
  uint32_t xsrc[G::nix_max];
#pragma unroll
  for (int q = 0; q < G::nix_max; ++q) {
    int i = (q * CW + cwave) * kWave + lane;
    if (i > xpos - 1) i = xpos - 1;
    const int ar = i / G::xp;
    const int pc = (i - ar * G::xp) ^ (ar & 15);
    xsrc[q] = static_cast<uint32_t>((static_cast<int64_t>(ar) * k + 8 * pc) * 2);
  }
  const uint8_t* const wbase = W + row0 * rb;
  const uint8_t* const xbase = reinterpret_cast<const uint8_t*>(x);

  // Copy instruction c (0 .. ndma - 1) of phase p: weight rounds first, then
  // activation rounds; a round with no copying lane is not issued.
  auto issue_one = [&](auto cc, int p) {
    constexpr int c = decltype(cc)::value;
    const uint32_t sb = smem + (p % kTSlots) * G::slot;
    if constexpr (c < G::niw) {
      const int i0 = (c * CW + cwave) * kWave;
      const uint8_t* ws = wbase + static_cast<int64_t>(p) * (PB * kBlockBytes);
      // Weights of at most two row tiles go non-temporal (each byte is read
      // once: 5120 x 17408 m = 10 16.3 -> 15.9 us, 7168 x 5120 8.0 -> 7.7 us);
      // with nine tiles the hint measured slower (34816 x 5120 m = 10:
      // 23.3 -> 24.4 us).
      if (i0 < wpos && i0 + lane < wpos) {
        if constexpr (T <= 2) dma16_sbase_nt(wsrc[c], ws, sb + i0 * 16);
        else dma16_sbase(wsrc[c], ws, sb + i0 * 16);
      }
    } else {
      constexpr int q = c - G::niw;
      const int i0 = (q * CW + cwave) * kWave;
      const uint8_t* xs = xbase + static_cast<int64_t>(p) * (G::phase_k * 2);
      if (i0 < xpos && i0 + lane < xpos) dma16_sbase(xsrc[q], xs, sb + G::wbytes + i0 * 16);
    }
  };
  auto issue = [&](int p) { unroll<0, G::ndma>([&](auto cc) { issue_one(cc, p); }); };

  // Lane roles: B side weight row r = lane % 16 and code dword g = lane / 16;
  // A side activation row a = lane % 16 (rows past m read row m - 1) and the
  // same g.  Byte offsets within a slot.
  const int r = lane & 15, g = lane >> 4;
  const uint32_t rs0 = r * G::wstride + wave * (G::jb * kBlockBytes);  // scale of block 0
  const uint32_t rg0 = rs0 + 4 * g;                                     // code dword g
  uint32_t xa[G::jb][2][AT];  // activation operand halves (elements 4g.. and 16 + 4g..)
#pragma unroll
  for (int t = 0; t < AT; ++t) {
    int ar = r + 16 * t;
    if (ar > m - 1) ar = m - 1;
    const int sw = ar & 15;
#pragma unroll
    for (int j = 0; j < G::jb; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pc = 4 * (wave * G::jb + j) + 2 * h + (g >> 1);
        xa[j][h][t] = G::wbytes + ar * (G::xp * 16) + 16 * (pc ^ sw) + 8 * (g & 1);
      }
  }
  const UnpackConsts kc = make_unpack_consts();
  bool inexact = false;  // a bf16 activation that fp16 does not hold exactly
  float4_t acc[T][AT];
#pragma unroll
  for (int i = 0; i < T; ++i)
#pragma unroll
    for (int t = 0; t < AT; ++t) acc[i][t] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int p, int pi) {
    const uint8_t* slot = tsm + (p % kTSlots) * G::slot;
    half8_t A[G::jb][AT];
#pragma unroll
    for (int j = 0; j < G::jb; ++j)
#pragma unroll
      for (int t = 0; t < AT; ++t) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(slot + xa[j][0][t]);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(slot + xa[j][1][t]);
        u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        if constexpr (XB) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t h = bf16x2_to_f16x2(a[e]);
            inexact |= !f16x2_holds_bf16x2(h, a[e]);
            a[e] = h;
          }
        }
        A[j][t] = __builtin_bit_cast(half8_t, a);
      }
    // Scale and code words of (row tile i, block j).  With one activation
    // tile every pair's words are read before the first product, so the
    // reads' latencies overlap one another instead of stalling each product
    // in turn (34816 x 5120 at m = 10: 24.9 -> 23.3 us; 5120 x 17408:
    // 17.2 -> 16.1 us); with two, each pair reads its own next to its product
    // (measured faster there, at the higher register count).
    uint32_t dw[T][G::jb], c0[T][G::jb], c1[T][G::jb];
    auto load_pair = [&](auto ii, auto jj) {
      constexpr int i = decltype(ii)::value;
      constexpr int j = decltype(jj)::value;
      constexpr int bo = i * 16 * G::wstride + j * kBlockBytes;
      dw[i][j] = *reinterpret_cast<const uint16_t*>(slot + rs0 + bo);
      if constexpr ((j & 1) == 0) {
        // even block: code bytes 4g .. 4g+3 are bytes 2..5 of the window at 4g
        c0[i][j] = *reinterpret_cast<const uint32_t*>(slot + rg0 + bo);
        c1[i][j] = *reinterpret_cast<const uint32_t*>(slot + rg0 + bo + 4);
      } else {
        // odd block: they are the aligned dword at 4g + 2
        c0[i][j] = *reinterpret_cast<const uint32_t*>(slot + rg0 + bo + 2);
        c1[i][j] = c0[i][j];
      }
    };
    if constexpr (AT == 1)
      unroll<0, T>([&](auto ii) { unroll<0, G::jb>([&](auto jj) { load_pair(ii, jj); }); });
    unroll<0, T>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      unroll<0, G::jb>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        // this tile's share of the copies of phase pi
        if (NP == 0 && pi >= 0) {
          unroll<0, G::dma_per_tile>([&](auto kk) {
            constexpr int c = (i * G::jb + j) * G::dma_per_tile + decltype(kk)::value;
            if constexpr (c < G::ndma) issue_one(TC<c>{}, pi);
          });
        }
        if constexpr (AT != 1) load_pair(ii, jj);
        const float d = half_bits_to_float(static_cast<uint16_t>(dw[i][j]));
        half8_t bw;
        if constexpr ((j & 1) == 0) bw = unpack8<2>(c0[i][j], c1[i][j], kc);
        else bw = unpack8<0>(c0[i][j], c0[i][j], kc);
#pragma unroll
        for (int t = 0; t < AT; ++t) {
          const float4_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              A[j][t], bw, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][t][e] = d * D[e] + acc[i][t][e];
        }
      });
    });
  };

  // Phase p: once only phase p + 1's copies are in flight (none when p is the
  // last phase) a copying wave's copies of p have landed; the barrier extends
  // that to every wave and frees the slot of phase p - 1, which phase p + 2's
  // copies then reuse.
  constexpr int kMaxInFlight = G::niw + G::nix_max;
  const int per_phase = cw + cx;
  if constexpr (NP == 0) {
    issue(0);
    if (nph > 1) issue(1);
    for (int p = 0; p < nph; ++p) {
      wait_vm_upto<kMaxInFlight>(p + 1 < nph ? per_phase : 0);
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      compute(p, p + 2 < nph ? p + 2 : -1);
      compiler_fence();
    }
  } else if (wave >= NW) {
    // copying waves: the phase's barrier once its copies have landed, then
    // the copies of phase p + 2
    issue(0);
    if (nph > 1) issue(1);
    for (int p = 0; p < nph; ++p) {
      wait_vm_upto<kMaxInFlight>(p + 1 < nph ? per_phase : 0);
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      if (p + 2 < nph) issue(p + 2);
    }
  } else {
    for (int p = 0; p < nph; ++p) {
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      if (p < 30) Q4_PHASE_MARK(1 + p);
      compute(p, -1);
      compiler_fence();
      if (p < 30) Q4_PHASE_MARK(32 + p);
    }
  }

  // Sum the eight waves' partial tiles (the ring is free once every wave has
  // passed this barrier), each output in wave order.  Lane l of a tile holds
  // its activation rows 4 (l / 16) .. + 3 for weight row l % 16.  From
  // kTileFragSum row tiles on, lanes whose four rows all lie past m do not
  // write, and one thread sums a lane's whole fragment (four float4 reads
  // per wave fewer than one thread per output; 34816 x 5120 at m = 10:
  // 24.3 -> 23.4 us).  With fewer tiles one thread per output measured
  // faster.
  __syncthreads();
  float4_t* red = reinterpret_cast<float4_t*>(tsm);
  if (wave < NW) {
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
      for (int t = 0; t < AT; ++t)
        if (T < kTileFragSum || 16 * t + 4 * (lane >> 4) < m)
          red[((i * AT + t) * NW + wave) * kWave + lane] = acc[i][t];
  }
  __syncthreads();
  if constexpr (T >= kTileFragSum) {
    for (int o = threadIdx.x; o < T * AT * kWave; o += G::lanes) {
      const int l = o & (kWave - 1);
      const int it = o / kWave;  // i AT + t
      const int i = it / AT, t = it - i * AT;
      const int a0 = 16 * t + 4 * (l >> 4), wr = l & 15;
      if (a0 >= m || 16 * i + wr >= rv) continue;
      float4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float4_t v = red[(it * NW + w) * kWave + l];
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[e] += v[e];
      }
      const int64_t row = row0 + 16 * i + wr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (a0 + e < m) {
          const int64_t off = static_cast<int64_t>(a0 + e) * n + row;
          if (y_f16) static_cast<half_t*>(y)[off] = static_cast<half_t>(sum[e]);
          else static_cast<float*>(y)[off] = sum[e];
        }
      }
    }
  } else {
    const float* rf = reinterpret_cast<const float*>(tsm);
    const int O = T * 16 * m;
    for (int o = threadIdx.x; o < O; o += G::lanes) {
      const int i = o / (16 * m);
      const int rem = o - i * 16 * m;
      const int ar = rem >> 4, wr = rem & 15;
      const int t = ar >> 4, aa = ar & 15;
      const int l = wr + 16 * (aa >> 2), e = aa & 3;
      const float* q = rf + (static_cast<int64_t>((i * AT + t) * NW) * kWave + l) * 4 + e;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += q[w * kWave * 4];
      const int64_t row = row0 + 16 * i + wr;
      if (16 * i + wr < rv) {
        const int64_t off = static_cast<int64_t>(ar) * n + row;
        if (y_f16) static_cast<half_t*>(y)[off] = static_cast<half_t>(sum);
        else static_cast<float*>(y)[off] = sum;
      }
    }
  }
  Q4_PHASE_MARK(63);
  Q4_PHASE_MARK_RT(62);
  if constexpr (XB) {
    if (workgroup_any_flag(inexact, reinterpret_cast<uint32_t*>(tsm)))
      gemv_exact_rows_bf16<NW + NP>(reinterpret_cast<const uint16_t*>(x), W, y, y_f16, m, n, k, row0,
                                    rv);
  }
}

template <int T, int AT, int PB, bool FULL, bool XB, int WR = 16 * T, int XR = 16 * AT,
          int NW = 8, int NP = 4>
hipError_t launch_tile_f(const void* x, const uint8_t* packed, void* y, bool y_f16, int m,
                         int64_t n, int64_t k, int rows, hipStream_t s) {
  using G = TileGeo<T, AT, PB, NW, NP, WR, XR>;
  static_assert(G::lds <= kTLdsMax, "LDS budget");
  const void* fn =
      reinterpret_cast<const void*>(&gemv_tile_kernel<T, AT, PB, FULL, NW, NP, XB, WR, XR>);
  static std::atomic<uint64_t> lds_allowed{0};
  const hipError_t e = allow_dynamic_lds(fn, kTLdsMax, lds_allowed);
  if (e != hipSuccess) return e;
  if (rows < 1 || rows > WR || m > XR) return hipErrorInvalidValue;
  const int64_t grid = (n + rows - 1) / rows;
  const half_t* xp = static_cast<const half_t*>(x);
  int yf = y_f16 ? 1 : 0;
  void* argv[] = {&xp, const_cast<const uint8_t**>(&packed), &y, &m, &n, &k, &yf, &rows};
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(G::lanes), argv,
                         static_cast<size_t>(G::lds), s);
}

template <int T, int AT, int PB, bool XB>
hipError_t launch_tile_t(const void* x, const uint8_t* packed, void* y, bool y_f16, int m,
                         int64_t n, int64_t k, int rows, hipStream_t s) {
  if (rows == 16 * T)
    return launch_tile_f<T, AT, PB, true, XB>(x, packed, y, y_f16, m, n, k, rows, s);
  return launch_tile_f<T, AT, PB, false, XB>(x, packed, y, y_f16, m, n, k, rows, s);
}

struct TilePlan {
  int T, AT, PB, rows;
  bool pair = false;  // two workgroups per compute unit (see kPairMaxRows)
};

// Five row tiles with two activation tiles (m > 16) fit the LDS ring only
// with at most this many weight rows per slot.
constexpr int kT5AT2Rows = 68;
// Up to this many activation rows, a slot's activation area holds only them
// (rows past m read row m - 1), which leaves room in three slots for nine
// row tiles: 144 rows per workgroup, so 34816 rows run as one round of 256
// workgroups instead of two rounds of 80-row workgroups (28.4 -> 25.5 us at
// m = 10).  Up to 16 rows, seven tiles fit.  Fewer, larger workgroups
// stream faster here: each one pays a start-up and a drain.
constexpr int kT9MaxM = 10;
constexpr int kT7MaxM = 16;
// Past one round of nine-tile workgroups (m <= 10, more than 144 rows per
// compute unit) the rows are instead split over two workgroups per compute
// unit, both resident at once: up to 112 rows each in 8-block phases (three
// slots of at most 26 KB), four computing and two copying waves.  A second
// round of large workgroups would leave most of the chip idle while it runs:
// 40000 x 5120 at m = 10 measured 40.5 -> 28.9 us, 49152 x 5120 41.3 ->
// 35.5 us, 40000 x 1024 15.7 -> 9.5 us; 57344 x 8192, where the large
// workgroups take three full rounds, 62.9 -> 61.5 us.
constexpr int kPairMaxRows = 112;
constexpr int kPairPB = 8;

// Rows per workgroup: whole 16-row tiles, enough for one workgroup per
// compute unit (capped where the LDS ring would not fit; larger matrices take
// several rounds).  With K long enough for eight or more phases the rows are
// instead spread evenly over every compute unit (the last tile partial): the
// streamed bytes per compute unit then dominate, and spreading lowers them.
// With fewer phases the extra workgroups' activation traffic and start-up
// cost more than that saves (measured at 5120 x 5120, m = 10 and 16).
TilePlan tile_plan(int m, int64_t n, int64_t k) {
  const int64_t cu = device_cu_count();
  TilePlan p;
  p.AT = m > 16 ? 2 : 1;
  int64_t tfull = ((n + 15) / 16 + cu - 1) / cu;  // tiles per workgroup for one round
  if (tfull < 1) tfull = 1;
  // Six or seven tiles for one round run on the seven-tile kernel (m <= 16);
  // more on the nine-tile kernel (m <= 10), in one round if they fit, and
  // past one round on two workgroups per compute unit (kPairMaxRows).  Past
  // one round, m = 11..16 keeps five tiles: a second round that holds few
  // seven-tile workgroups measured slower than two rounds of five.
  int tmax = 5;
  if (p.AT == 2) tmax = 4;
  else if (tfull <= 7 && m <= kT7MaxM) tmax = 7;
  else if (m <= kT9MaxM) tmax = 9;
  if (tmax == 9 && tfull > 9 && k % (kPairPB * kQK) == 0) {
    int64_t rows = (n + 2 * cu - 1) / (2 * cu);
    rows = (rows + 3) / 4 * 4;
    if (rows <= kPairMaxRows) {
      p.PB = kPairPB;
      p.rows = static_cast<int>(rows);
      p.T = static_cast<int>((rows + 15) / 16);  // 5 .. 7
      p.pair = true;
      return p;
    }
  }
  const bool wide = tfull > tmax;
  if (tfull > tmax) tfull = tmax;
  p.PB = p.AT == 1 && tfull <= 2 && k % 1024 == 0 ? 32 : 16;
  int64_t rows = 16 * tfull;
  const int64_t nph = k / (p.PB * kQK);
  if (nph >= 8) {
    const int64_t spread = (n + cu - 1) / cu;
    if (spread < rows) rows = spread;
  }
  // m > 16 with more than 64 rows per compute unit: up to 68 rows in five
  // tiles (a slot sized for 68 weight rows) keeps 17408 rows in one round of
  // 256 workgroups instead of 272 (a second round for the last 16).
  if (p.AT == 2 && wide) {
    const int64_t spread = (n + cu - 1) / cu;
    rows = spread < kT5AT2Rows ? spread : kT5AT2Rows;
  }
  p.rows = static_cast<int>(rows);
  p.T = static_cast<int>((rows + 15) / 16);
  // six to nine tiles run on the seven- or nine-tile kernel (rows past p.rows
  // are not copied)
  if (p.T > 5) p.T = p.T <= 7 ? 7 : 9;
  return p;
}

template <int AT, int PB, bool XB>
hipError_t launch_tile_tt(const TilePlan& p, const void* x, const uint8_t* packed, void* y,
                          bool y_f16, int m, int64_t n, int64_t k, hipStream_t s) {
  switch (p.T) {
    case 1: return launch_tile_t<1, AT, PB, XB>(x, packed, y, y_f16, m, n, k, p.rows, s);
    case 2: return launch_tile_t<2, AT, PB, XB>(x, packed, y, y_f16, m, n, k, p.rows, s);
    case 3: return launch_tile_t<3, AT, PB, XB>(x, packed, y, y_f16, m, n, k, p.rows, s);
    case 4: return launch_tile_t<4, AT, PB, XB>(x, packed, y, y_f16, m, n, k, p.rows, s);
    case 7:
      if constexpr (AT == 1 && PB == 16) {
        if (p.rows == 112)
          return launch_tile_f<7, 1, 16, true, XB, 112, kT7MaxM>(x, packed, y, y_f16, m, n, k,
                                                                 p.rows, s);
        return launch_tile_f<7, 1, 16, false, XB, 112, kT7MaxM>(x, packed, y, y_f16, m, n, k,
                                                                p.rows, s);
      }
      return hipErrorInvalidValue;
    case 9:
      if constexpr (AT == 1 && PB == 16) {
        if (p.rows == 144)
          return launch_tile_f<9, 1, 16, true, XB, 144, kT9MaxM>(x, packed, y, y_f16, m, n, k,
                                                                 p.rows, s);
        return launch_tile_f<9, 1, 16, false, XB, 144, kT9MaxM>(x, packed, y, y_f16, m, n, k,
                                                                p.rows, s);
      }
      return hipErrorInvalidValue;
    default:
      if constexpr (AT == 1 && PB == 16)
        return launch_tile_t<5, AT, PB, XB>(x, packed, y, y_f16, m, n, k, p.rows, s);
      if constexpr (AT == 2 && PB == 16)
        return launch_tile_f<5, 2, 16, false, XB, kT5AT2Rows>(x, packed, y, y_f16, m, n, k,
                                                              p.rows, s);
      return hipErrorInvalidValue;
  }
}

template <bool XB>
hipError_t launch_tile_x(const TilePlan& p, const void* x, const uint8_t* packed, void* y,
                         bool y_f16, int m, int64_t n, int64_t k, hipStream_t s) {
  if (p.pair) {
    // two resident workgroups per compute unit: 4 computing + 2 copying waves
    switch (p.T) {
      case 5:
        return launch_tile_f<5, 1, kPairPB, false, XB, 80, kT9MaxM, 4, 2>(x, packed, y, y_f16, m, n,
                                                                           k, p.rows, s);
      case 6:
        return launch_tile_f<6, 1, kPairPB, false, XB, 96, kT9MaxM, 4, 2>(x, packed, y, y_f16, m, n,
                                                                           k, p.rows, s);
      case 7:
        return launch_tile_f<7, 1, kPairPB, false, XB, 112, kT9MaxM, 4, 2>(x, packed, y, y_f16, m,
                                                                            n, k, p.rows, s);
      default:
        return hipErrorInvalidValue;
    }
  }
  if (p.AT == 2) return launch_tile_tt<2, 16, XB>(p, x, packed, y, y_f16, m, n, k, s);
  if (p.PB == 32) {
    if (p.T == 1) return launch_tile_t<1, 1, 32, XB>(x, packed, y, y_f16, m, n, k, p.rows, s);
    return launch_tile_t<2, 1, 32, XB>(x, packed, y, y_f16, m, n, k, p.rows, s);
  }
  return launch_tile_tt<1, 16, XB>(p, x, packed, y, y_f16, m, n, k, s);
}

}  // namespace

bool gemv_tile_supports(int m, int64_t k) { return m >= 1 && m <= 32 && k > 0 && k % 512 == 0; }

hipError_t launch_gemv_tile(const void* x, bool x_bf16, const uint8_t* packed, void* y,
                            bool y_f16, int m, int64_t n, int64_t k, hipStream_t s) {
  const TilePlan p = tile_plan(m, n, k);
  if (x_bf16) return launch_tile_x<true>(p, x, packed, y, y_f16, m, n, k, s);
  return launch_tile_x<false>(p, x, packed, y, y_f16, m, n, k, s);
}

}  // namespace q4

#ifdef Q4_PHASE_TRACE
// Sets (or, with nullptr, clears) the buffer the measurement build's tile
// kernels record their phase clocks into; returns 0, or 1 on a HIP error.
extern "C" int q4_phase_trace_set(void* buf) {
  return hipMemcpyToSymbol(HIP_SYMBOL(q4::g_phase_trace), &buf, sizeof(buf)) == hipSuccess ? 0 : 1;
}
#endif
