// libq4host: the host-CPU twin of the batched-decode GEMV (include/q4_host.h).
//
// "Vertical disaggregation: maximizing throughput on heterogeneous silicon",
// section "Every cycle counts: custom kernels": the CPU backend reads the same
// Q4_0 bytes as the GPU backend and its output is deterministic.  The kernel
// stages that section names map onto AVX2 as follows, per 18-byte block:
//   nibble unpack -- one 16-byte load of the codes; low nibbles (elements
//                    0..15) by a mask, high nibbles (elements 16..31) by a
//                    16-bit shift and the same mask; minus 8; widened to four
//                    eight-lane fp32 vectors (exact: integers -8..7);
//   scale         -- those vectors times the block's fp16 scale widened to
//                    fp32: w = (q - 8) d, exact in fp32;
//   dot product   -- four eight-wide fused multiply-adds of the activations
//                    with w into a per-output eight-lane fp32 accumulator;
//   batch decode  -- the unpacked block serves every activation row, and four
//                    weight rows share each activation load (fp16 activations
//                    are widened once per call into a host buffer).
// Each output's lanes accumulate blocks in k order and are summed in a fixed
// pairwise order at the end; one thread owns each output, so the bits do not
// depend on the thread count.  Rows are split over std::threads in contiguous
// ranges.  The vector code is compiled for AVX2 + FMA + F16C through function
// target attributes and is entered only after a run-time CPU check, so the
// library loads on any x86-64 host.
#include "q4_host.h"

#include <immintrin.h>
#include <sched.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr int64_t kQK = Q4_QK;
constexpr int64_t kBlockBytes = Q4_BLOCK_BYTES;
constexpr int kMaxM = Q4_GEMV_MAX_M;
constexpr int kRows = 4;  // weight rows sharing each activation load

#define Q4_HOST_TARGET __attribute__((target("avx2,fma,f16c")))

bool cpu_has_features() {
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
         __builtin_cpu_supports("f16c");
}

// The block's weights w = (q - 8) d in four fp32 vectors (elements 0-7,
// 8-15, 16-23, 24-31); exact, since (q - 8) has at most 4 significant bits
// and d at most 11.
struct Unpacked {
  __m256 w[4];
};

Q4_HOST_TARGET inline Unpacked unpack_block(const uint8_t* blk) {
  Unpacked u;
  uint16_t dbits;
  std::memcpy(&dbits, blk, 2);
  const __m256 d = _mm256_set1_ps(_cvtsh_ss(dbits));
  const __m128i mask = _mm_set1_epi8(0x0F);
  const __m128i eight = _mm_set1_epi8(8);
  const __m128i c = _mm_loadu_si128(reinterpret_cast<const __m128i*>(blk + 2));
  const __m128i lo = _mm_sub_epi8(_mm_and_si128(c, mask), eight);
  const __m128i hi = _mm_sub_epi8(_mm_and_si128(_mm_srli_epi16(c, 4), mask), eight);
  u.w[0] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(lo)), d);
  u.w[1] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_unpackhi_epi64(lo, lo))), d);
  u.w[2] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(hi)), d);
  u.w[3] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_unpackhi_epi64(hi, hi))), d);
  return u;
}

// fp16 activations widened exactly to fp32 (F16C), once per call.
Q4_HOST_TARGET void widen_x(const uint16_t* x, float* out, int64_t count) {
  int64_t i = 0;
  for (; i + 8 <= count; i += 8)
    _mm256_storeu_ps(out + i, _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(x + i))));
  for (; i < count; ++i) out[i] = _cvtsh_ss(x[i]);
}

// acc + x . w over one block, lane-wise, in element order.
Q4_HOST_TARGET inline __m256 block_fma(const __m256 xv[4], const __m256 w[4], __m256 acc) {
  acc = _mm256_fmadd_ps(xv[0], w[0], acc);
  acc = _mm256_fmadd_ps(xv[1], w[1], acc);
  acc = _mm256_fmadd_ps(xv[2], w[2], acc);
  return _mm256_fmadd_ps(xv[3], w[3], acc);
}

// Fixed-order sum of the eight lanes: ((0+1)+(2+3)) + ((4+5)+(6+7)).
Q4_HOST_TARGET inline float lane_sum(__m256 a) {
  alignas(32) float t[8];
  _mm256_store_ps(t, a);
  return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

Q4_HOST_TARGET inline void store_y(void* y, bool yh, int64_t off, float v) {
  if (yh) static_cast<uint16_t*>(y)[off] = _cvtss_sh(v, _MM_FROUND_TO_NEAREST_INT);
  else static_cast<float*>(y)[off] = v;
}

// R (1 to 4) consecutive weight rows starting at r, all m activation rows
// (fp32 x).
template <int R>
Q4_HOST_TARGET void rows_kernel(const float* x, const uint8_t* W, void* y, bool yh, int m, int64_t n,
                                int64_t k, int64_t r) {
  const int64_t nb = k / kQK;
  const int64_t rb = nb * kBlockBytes;
  __m256 acc[R][kMaxM];
  for (int j = 0; j < R; ++j)
    for (int i = 0; i < m; ++i) acc[j][i] = _mm256_setzero_ps();
  for (int64_t b = 0; b < nb; ++b) {
    Unpacked u[R];
    for (int j = 0; j < R; ++j) u[j] = unpack_block(W + (r + j) * rb + b * kBlockBytes);
    for (int i = 0; i < m; ++i) {
      const float* xp = x + static_cast<int64_t>(i) * k + b * kQK;
      __m256 xv[4];
      for (int e = 0; e < 4; ++e) xv[e] = _mm256_loadu_ps(xp + 8 * e);
      for (int j = 0; j < R; ++j) acc[j][i] = block_fma(xv, u[j].w, acc[j][i]);
    }
  }
  for (int j = 0; j < R; ++j)
    for (int i = 0; i < m; ++i) store_y(y, yh, static_cast<int64_t>(i) * n + r + j, lane_sum(acc[j][i]));
}

Q4_HOST_TARGET void row_range(const float* x, const uint8_t* W, void* y, bool yh, int m, int64_t n,
                              int64_t k, int64_t r0, int64_t r1) {
  int64_t r = r0;
  for (; r + kRows <= r1; r += kRows) rows_kernel<kRows>(x, W, y, yh, m, n, k, r);
  for (; r < r1; ++r) rows_kernel<1>(x, W, y, yh, m, n, k, r);
}

int affinity_cpus() {
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    const int c = CPU_COUNT(&set);
    if (c > 0) return c;
  }
  const unsigned h = std::thread::hardware_concurrency();
  return h > 0 ? static_cast<int>(h) : 1;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

size_t dtype_size(int dt) { return dt == Q4_F16 ? 2 : 4; }

}  // namespace

extern "C" {

int q4_host_abi_version(void) { return Q4_HOST_ABI_VERSION; }

int q4_host_default_threads(void) { return affinity_cpus(); }

q4_status q4_host_gemv(const void* x, int x_dtype, const void* packed, void* y, int y_dtype,
                       int64_t m, int64_t n, int64_t k, int threads) {
  if (!x || !packed || !y) return Q4_ERR_INVALID_ARG;
  if (m < 1 || m > kMaxM || n < 1 || k < kQK || k % kQK != 0) return Q4_ERR_SHAPE;
  if (n > (int64_t{1} << 40) / k) return Q4_ERR_SHAPE;
  if ((x_dtype != Q4_F32 && x_dtype != Q4_F16) || (y_dtype != Q4_F32 && y_dtype != Q4_F16))
    return Q4_ERR_DTYPE;
  const size_t ybytes = static_cast<size_t>(m) * n * dtype_size(y_dtype);
  const size_t xbytes = static_cast<size_t>(m) * k * dtype_size(x_dtype);
  const size_t wbytes = static_cast<size_t>(n) * (k / kQK) * kBlockBytes;
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, packed, wbytes))
    return Q4_ERR_INVALID_ARG;
  if (!cpu_has_features()) return Q4_ERR_UNSUPPORTED;

  const uint8_t* W = static_cast<const uint8_t*>(packed);
  const bool yh = y_dtype == Q4_F16;
  const int mi = static_cast<int>(m);
  // fp16 activations are widened once into a host buffer of m * k floats.
  std::vector<float> xw;
  const float* xf = static_cast<const float*>(x);
  if (x_dtype == Q4_F16) {
    try {
      xw.resize(static_cast<size_t>(m) * k);
    } catch (...) {
      return Q4_ERR_INVALID_ARG;
    }
    widen_x(static_cast<const uint16_t*>(x), xw.data(), m * k);
    xf = xw.data();
  }
  // Threads own contiguous ranges of row groups.
  const int64_t groups = (n + kRows - 1) / kRows;
  int64_t t = threads > 0 ? threads : affinity_cpus();
  t = std::max<int64_t>(1, std::min(t, groups));
  auto work = [&](int64_t i) {
    const int64_t r0 = std::min(n, kRows * (groups * i / t));
    const int64_t r1 = std::min(n, kRows * (groups * (i + 1) / t));
    row_range(xf, W, y, yh, mi, n, k, r0, r1);
  };
  std::vector<std::thread> pool;
  int64_t inline_from = t - 1;  // ranges the calling thread runs
  try {
    pool.reserve(static_cast<size_t>(t - 1));
    for (int64_t i = 0; i < t - 1; ++i) {
      pool.emplace_back(work, i);
    }
  } catch (...) {
    inline_from = static_cast<int64_t>(pool.size());  // threads the system refused: run here
  }
  for (int64_t i = inline_from; i < t; ++i) work(i);
  for (auto& th : pool) th.join();
  return Q4_OK;
}

}  // extern "C"
