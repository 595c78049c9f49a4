// Sanitizer driver for the host-CPU twin (libq4host, include/q4_host.h): runs
// q4_host_gemv over many shapes, dtypes and thread counts on seeded packed
// bytes and checks that every thread count gives the single-thread bits (the
// header's determinism promise), then every argument check.  Built and run by
// tests/test_sanitizers.py under AddressSanitizer + UndefinedBehaviorSanitizer
// and under ThreadSanitizer; a sanitizer report or a mismatch exits non-zero.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "q4_host.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
  }
}

// fp16 bits of a modest positive or negative scale (exponent 2^-8 .. 2^1).
uint16_t scale_bits(std::mt19937& g) {
  const uint16_t e = static_cast<uint16_t>(7 + g() % 10), mant = static_cast<uint16_t>(g() & 0x3FF);
  return static_cast<uint16_t>(((g() & 1) << 15) | (e << 10) | mant);
}

void run_shape(std::mt19937& g, int m, int n, int k, int xdt, int ydt) {
  const int nb = k / 32;
  std::vector<uint8_t> packed(static_cast<size_t>(n) * nb * 18);
  for (int r = 0; r < n; ++r)
    for (int b = 0; b < nb; ++b) {
      uint8_t* blk = &packed[(static_cast<size_t>(r) * nb + b) * 18];
      const uint16_t d = scale_bits(g);
      std::memcpy(blk, &d, 2);
      for (int i = 0; i < 16; ++i) blk[2 + i] = static_cast<uint8_t>(g());
    }
  const size_t xe = static_cast<size_t>(m) * k, ye = static_cast<size_t>(m) * n;
  std::vector<uint8_t> x(xe * (xdt == Q4_F32 ? 4 : 2));
  for (size_t i = 0; i < xe; ++i) {
    if (xdt == Q4_F32) {
      const float v = static_cast<float>(static_cast<int>(g() % 2001) - 1000) / 256.0f;
      std::memcpy(&x[4 * i], &v, 4);
    } else {
      const uint16_t h = static_cast<uint16_t>(((g() & 1) << 15) | ((10 + g() % 8) << 10) | (g() & 0x3FF));
      std::memcpy(&x[2 * i], &h, 2);
    }
  }
  const size_t yb = ye * (ydt == Q4_F32 ? 4 : 2);
  std::vector<uint8_t> y1(yb, 0xCD), yt(yb, 0xCD);
  expect(q4_host_gemv(x.data(), xdt, packed.data(), y1.data(), ydt, m, n, k, 1) == Q4_OK, "1 thread");
  for (int t : {2, 3, 8, 64}) {
    std::fill(yt.begin(), yt.end(), 0xCD);
    expect(q4_host_gemv(x.data(), xdt, packed.data(), yt.data(), ydt, m, n, k, t) == Q4_OK, "threads");
    expect(std::memcmp(y1.data(), yt.data(), yb) == 0, "thread count changed the bits");
  }
}

}  // namespace

int main() {
  std::mt19937 g(12345);
  const int shapes[][3] = {{1, 1, 32}, {1, 7, 96}, {4, 129, 512}, {5, 64, 1056}, {16, 300, 2048},
                           {32, 37, 544}, {3, 513, 5120}};
  for (const auto& s : shapes)
    for (int xdt : {Q4_F16, Q4_F32})
      for (int ydt : {Q4_F16, Q4_F32}) run_shape(g, s[0], s[1], s[2], xdt, ydt);

  // argument checks (return before any work)
  std::vector<uint8_t> buf(1 << 16);
  uint8_t* x = buf.data();
  uint8_t* p = buf.data() + 8192;
  uint8_t* y = buf.data() + 32768;
  expect(q4_host_gemv(nullptr, Q4_F16, p, y, Q4_F16, 1, 8, 32, 1) == Q4_ERR_INVALID_ARG, "null x");
  expect(q4_host_gemv(x, Q4_F16, nullptr, y, Q4_F16, 1, 8, 32, 1) == Q4_ERR_INVALID_ARG, "null packed");
  expect(q4_host_gemv(x, Q4_F16, p, nullptr, Q4_F16, 1, 8, 32, 1) == Q4_ERR_INVALID_ARG, "null y");
  expect(q4_host_gemv(x, Q4_F16, p, y, Q4_F16, 0, 8, 32, 1) == Q4_ERR_SHAPE, "m = 0");
  expect(q4_host_gemv(x, Q4_F16, p, y, Q4_F16, 33, 8, 32, 1) == Q4_ERR_SHAPE, "m = 33");
  expect(q4_host_gemv(x, Q4_F16, p, y, Q4_F16, 1, 8, 48, 1) == Q4_ERR_SHAPE, "k % 32");
  expect(q4_host_gemv(x, 7, p, y, Q4_F16, 1, 8, 32, 1) == Q4_ERR_DTYPE, "x dtype");
  expect(q4_host_gemv(x, Q4_F16, p, y, Q4_BF16, 1, 8, 32, 1) == Q4_ERR_DTYPE, "y dtype");
  expect(q4_host_gemv(x, Q4_F16, p, x, Q4_F16, 1, 8, 32, 1) == Q4_ERR_INVALID_ARG, "y over x");
  expect(q4_host_gemv(x, Q4_F16, p, p + 16, Q4_F16, 1, 8, 32, 1) == Q4_ERR_INVALID_ARG, "y over packed");
  std::printf("host twin driver: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
