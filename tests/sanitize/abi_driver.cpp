// Sanitizer driver for libq4's host-side code (include/q4.h): every argument
// check of every entry point, and the size helpers and launch planner over a
// sweep of shapes, with no GPU call reached (each case returns before
// anything is launched).  Built and run by tests/test_sanitizers.py with the
// library's sources compiled under AddressSanitizer + UndefinedBehaviorSanitizer
// for the host; a sanitizer report or a wrong status exits non-zero.
#include <cstdint>
#include <cstdio>

#include "q4.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
  }
}

void* at(uintptr_t a) { return reinterpret_cast<void*>(a); }

}  // namespace

int main() {
  const uintptr_t A = 0x10000, B = 0x20000000, C = 0x40000000, W = 0x60000000;
  expect(q4_abi_version() == Q4_ABI_VERSION, "abi version");
  for (int s = -1; s < 12; ++s) expect(q4_status_string(s) != nullptr, "status string");
  // sizes and plans over a sweep of shapes (the planner's arithmetic)
  const int64_t ms[] = {1, 7, 64, 255, 256, 300, 1023, 1024, 2048, 4096, 8191};
  const int64_t ns[] = {1, 4, 100, 1024, 5120, 7168, 17408, 34816};
  const int64_t ks[] = {32, 64, 96, 512, 1024, 1088, 5120, 17408, 65536};
  for (int64_t m : ms)
    for (int64_t n : ns)
      for (int64_t k : ks) {
        const size_t p = q4_packed_size(n, k);
        expect(p == static_cast<size_t>(n) * (k / 32) * 18, "packed size");
        const size_t w16 = q4_gemm_workspace_size(m, n, k);
        const size_t wb = q4_gemm_workspace_size_dt(m, n, k, Q4_BF16);
        expect(wb >= w16 + static_cast<size_t>(m) * k * 2, "bf16 workspace");
        expect(q4_gemm_workspace_size_dt(m, n, k, Q4_F32) == 0, "fp32 workspace");
      }
  expect(q4_packed_size(1, 48) == 0 && q4_packed_size(0, 32) == 0, "invalid packed size");
  // argument checks
  expect(q4_quantize(nullptr, Q4_F32, 4, 32, at(B), nullptr) == Q4_ERR_INVALID_ARG, "q null");
  expect(q4_quantize(at(A), Q4_F32, 4, 48, at(B), nullptr) == Q4_ERR_SHAPE, "q shape");
  expect(q4_quantize(at(A), 9, 4, 32, at(B), nullptr) == Q4_ERR_DTYPE, "q dtype");
  expect(q4_quantize(at(A + 4), Q4_F32, 4, 32, at(B), nullptr) == Q4_ERR_ALIGNMENT, "q align");
  expect(q4_quantize(at(A), Q4_F32, 4, 32, at(A + 256), nullptr) == Q4_ERR_INVALID_ARG, "q overlap");
  expect(q4_gemv(at(A), Q4_F16, at(B), at(C), Q4_F16, 33, 8, 32, nullptr) == Q4_ERR_SHAPE, "v m");
  expect(q4_gemv(at(A), Q4_F16, at(B), at(C), Q4_BF16, 1, 8, 32, nullptr) == Q4_ERR_DTYPE, "v y");
  expect(q4_gemv(at(A), Q4_F16, at(B), at(A), Q4_F16, 1, 8, 32, nullptr) == Q4_ERR_INVALID_ARG, "v ov");
  expect(q4_gemv(at(A), Q4_F16, at(B), at(C), Q4_F16, 1, 1, (int64_t(1) << 24) + 32, nullptr) ==
             Q4_ERR_SHAPE, "v k limit");
  expect(q4_gemm(at(A), 7, at(B), at(C), Q4_F16, 64, 8, 32, nullptr, 0, nullptr) == Q4_ERR_DTYPE, "g dt");
  expect(q4_gemm(at(A + 8), Q4_F16, at(B), at(C), Q4_F16, 64, 8, 32, nullptr, 0, nullptr) ==
             Q4_ERR_ALIGNMENT, "g align");
  const size_t need = q4_gemm_workspace_size_dt(64, 8, 32, Q4_BF16);
  expect(q4_gemm(at(A), Q4_BF16, at(B), at(C), Q4_F16, 64, 8, 32, nullptr, 0, nullptr) ==
             Q4_ERR_WORKSPACE, "g ws");
  expect(q4_gemm(at(A), Q4_BF16, at(B), at(C), Q4_F16, 64, 8, 32, at(W), need - 1, nullptr) ==
             Q4_ERR_WORKSPACE, "g ws small");
  expect(q4_gemm(at(A), Q4_BF16, at(B), at(C), Q4_F16, 64, 8, 32, at(A), need, nullptr) ==
             Q4_ERR_INVALID_ARG, "g ws overlap");
  expect(q4_gemm_noalloc(at(A), Q4_BF16, at(B), at(C), Q4_F16, 8192, 64, 8192, nullptr) ==
             Q4_ERR_SCRATCH, "noalloc scratch");
  expect(q4_gemm_noalloc(nullptr, Q4_F16, at(B), at(C), Q4_F16, 64, 8, 32, nullptr) ==
             Q4_ERR_INVALID_ARG, "noalloc null");
  std::printf("abi driver: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
