/*
 * libq4host -- the host-CPU twin of q4_gemv, over the same packed Q4_0 bytes.
 *
 * "Vertical disaggregation: maximizing throughput on heterogeneous silicon",
 * section "Every cycle counts: custom kernels": the serving system runs decode
 * on CPUs (its kernels there target Zen3 / AVX2) as well as on GPUs, under one
 * hard rule -- both backends read one shared Q4_0 weight copy and give
 * deterministic output, so a session can move between them at the
 * prefill/decode boundary without recomputation.  This library is the CPU side
 * of the batched-decode GEMV: it reads the packed buffer that q4_quantize
 * writes (format stated in q4.h), byte for byte, from host memory.
 *
 * It is a separate backend, not a fallback: libq4 (the GPU library) never calls
 * it and it never calls libq4; a caller picks the backend explicitly.
 *
 * Arithmetic: every weight is dequantised exactly to fp32, w = (q - 8) * d,
 * and y[i][r] = sum_k x[i][k] * w[r][k] is accumulated with eight-lane fp32
 * fused multiply-adds (lane l takes the elements k = l mod 8, in k order); the
 * eight lanes are summed in a fixed order at the end and the result is rounded
 * once to the output dtype.  Every output is computed by one
 * thread in that fixed order, so the result does not depend on the thread
 * count: identical inputs give identical bits.
 */
#ifndef LIBQ4_Q4_HOST_H
#define LIBQ4_Q4_HOST_H

#include "q4.h"

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_HOST_ABI_VERSION 1

/* Version of this ABI (Q4_HOST_ABI_VERSION). */
int q4_host_abi_version(void);

/* Threads a call with threads <= 0 uses: the CPUs this process may run on. */
int q4_host_default_threads(void);

/* Batched-decode GEMV on the host: y[m][n] = x[m][k] . dequant(packed)^T for
 * 1 <= m <= Q4_GEMV_MAX_M.  All pointers are host pointers owned by the
 * caller; no alignment is required.  x is row-major [m][k] of dtype x_dtype
 * (Q4_F32 or Q4_F16), packed is the [n][k/32] x 18-byte Q4_0 buffer, y is
 * row-major [m][n] of dtype y_dtype (Q4_F32 or Q4_F16; fp16 rounds to nearest
 * even).  `threads` worker threads split the rows (<= 0: the default above);
 * the call returns when y is complete.  Errors, checked before any work:
 * Q4_ERR_INVALID_ARG (NULL pointer, y overlapping x or packed), Q4_ERR_SHAPE
 * (m outside 1..32, n < 1, k < 32, k % 32 != 0, n * k >= 2^40), Q4_ERR_DTYPE,
 * Q4_ERR_UNSUPPORTED (the CPU lacks AVX2, FMA or F16C). */
q4_status q4_host_gemv(const void *x, int x_dtype, const void *packed, void *y,
                       int y_dtype, int64_t m, int64_t n, int64_t k, int threads);

#ifdef __cplusplus
}
#endif

#endif /* LIBQ4_Q4_HOST_H */
