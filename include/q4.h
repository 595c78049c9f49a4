/*
 * libq4 -- Q4_0 block-quantised linear layers on AMD Instinct MI355X (gfx950).
 *
 * The C ABI of the library.  Plain pointers and sizes only; no HIP or torch
 * types appear in a signature (a stream is passed as an opaque pointer that
 * is a hipStream_t).
 *
 * The operation
 * -------------
 * "Vertical disaggregation: maximizing throughput on heterogeneous silicon",
 * section "Every cycle counts: custom kernels": the CPU and GPU backends share
 * one Q4_0 weight copy, output is deterministic, and the kernel stages are
 * nibble unpack, dot product, scale application, batched decode and a GPU
 * path onto matrix cores for prefill.  The format itself is not printed on
 * the page; this library fixes it as:
 *
 *   - a weight W[n][k] (row-major, n output features, k input features) is
 *     split along k into blocks of 32 (k must be a multiple of 32);
 *   - each block is 18 bytes: a 2-byte little-endian IEEE fp16 scale d, then
 *     16 code bytes; byte i holds the 4-bit code q of element i in its low
 *     nibble and of element i+16 in its high nibble;
 *   - a weight decodes as w = (q - 8) * d;
 *   - the packed buffer is n rows of k/32 consecutive blocks, rows
 *     contiguous: n * (k/32) * 18 bytes, no padding.
 *
 * Quantiser: m is the block element of largest magnitude (the first on a
 * tie); d = fp16(m / -8) rounded to nearest even, subnormals kept;
 * q = min(15, trunc(x / d + 8.5)) with x / d a correctly rounded fp32 division
 * by the fp16 scale widened to fp32 and the + 8.5 an fp32 addition; every q is
 * 8 when d is zero.
 *
 * Matmul: y[m][n] = sum_k x[m][k] * w[n][k] (x row-major [m][k], y row-major
 * [m][n]), accumulated in fp32.  Results are deterministic: identical inputs,
 * shapes and dtypes on the same device and build give identical bits (no
 * atomics, fixed reduction order).
 *
 * Conventions for every entry point
 * ---------------------------------
 *   - all data pointers are device pointers owned by the caller; the library
 *     never allocates, frees or synchronises, keeps no state, and is safe to
 *     call from several host threads;
 *   - every call is asynchronous on `stream` (NULL = the null stream); errors
 *     detected on the host return before anything is launched; a failed
 *     launch returns Q4_ERR_HIP; faults during execution surface at the
 *     caller's next synchronisation, as for any HIP library;
 *   - every data pointer must be 16-byte aligned (Q4_ERR_ALIGNMENT) and
 *     non-NULL (Q4_ERR_INVALID_ARG); outputs must not overlap inputs
 *     (Q4_ERR_INVALID_ARG);
 *   - shapes: n >= 1, m >= 1, k >= 32 and k % 32 == 0, and n * k below 2^40
 *     (Q4_ERR_SHAPE); for q4_gemv and q4_gemm also k <= 2^24 (the kernels
 *     address a tile's activation rows with 32-bit per-lane byte offsets);
 *   - inputs must be finite; weights must satisfy |w| < 65520 * 8 so that d
 *     is finite.  This is not checked on the device.
 */
#ifndef LIBQ4_Q4_H
#define LIBQ4_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_ABI_VERSION 1
#define Q4_QK 32            /* weights per block */
#define Q4_BLOCK_BYTES 18   /* bytes per block */
#define Q4_GEMV_MAX_M 32    /* largest batch accepted by q4_gemv */

/* An opaque hipStream_t. */
typedef struct ihipStream_t *q4_stream_t;

typedef enum q4_status {
  Q4_OK = 0,
  Q4_ERR_INVALID_ARG = 1, /* NULL pointer, overlapping buffers */
  Q4_ERR_SHAPE = 2,       /* m, n or k out of range, k % 32 != 0 */
  Q4_ERR_DTYPE = 3,       /* dtype code not supported by this call */
  Q4_ERR_ALIGNMENT = 4,   /* a pointer is not 16-byte aligned */
  Q4_ERR_HIP = 5,         /* the HIP runtime refused a launch */
  Q4_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
  Q4_ERR_UNSUPPORTED = 7, /* the host CPU lacks an instruction set the call needs
                             (q4_host.h) */
  Q4_ERR_SCRATCH = 8      /* the call needs more scratch than q4_gemm_noalloc's
                             fixed per-device array holds */
} q4_status;

typedef enum q4_dtype {
  Q4_F32 = 0, /* IEEE binary32 */
  Q4_F16 = 1, /* IEEE binary16 */
  Q4_BF16 = 2 /* bfloat16: the upper 16 bits of a binary32 pattern; accepted
                 for weights and activations, not for outputs */
} q4_dtype;

/* Version of this ABI (Q4_ABI_VERSION). */
int q4_abi_version(void);

/* Static, NUL-terminated description of a status code; never NULL. */
const char *q4_status_string(int status);

/* Size in bytes of a packed [n][k] Q4_0 weight: n * (k/32) * 18.
 * Returns 0 when the shape is invalid (n < 1, k < 32, k % 32 != 0). */
size_t q4_packed_size(int64_t n, int64_t k);

/* Quantise a row-major [n][k] weight `w` of dtype `w_dtype` (Q4_F32, Q4_F16
 * or Q4_BF16; fp16 and bf16 are widened exactly to fp32 first) into `packed`,
 * which must hold q4_packed_size(n, k) bytes.  The result is bit-identical to
 * the rule stated at the top of this header.  Reads 4 (fp32) or 2 (fp16,
 * bf16) bytes and writes 0.5625 bytes per weight. */
q4_status q4_quantize(const void *w, int w_dtype, int64_t n, int64_t k,
                      void *packed, q4_stream_t stream);

/* Batched-decode GEMV: y[m][n] = x[m][k] . dequant(packed)^T for
 * 1 <= m <= Q4_GEMV_MAX_M (the page's batched decode stage).  x is Q4_F32,
 * Q4_F16 or Q4_BF16, y is Q4_F32 or Q4_F16.  Every output is the fp32 sum
 * over blocks of d times the block dot product of x with (q - 8), rounded
 * once to the output dtype.  The block products take the codes as exact
 * integers q - 8, so each product x (q - 8) is exact and the error is fp32
 * summation error relative to sum |x w|, for every in-domain input.  bf16
 * x with k a multiple of 512 is converted to fp16 inside the kernel (round
 * to nearest even); a workgroup whose conversion was inexact anywhere (a
 * value beyond fp16's range or off its subnormal grid) recomputes its
 * outputs with x widened exactly to fp32, so the result is exact for every
 * bf16 value; other bf16 shapes are widened exactly to fp32.  Streams each
 * packed byte from memory once per call. */
q4_status q4_gemv(const void *x, int x_dtype, const void *packed, void *y,
                  int y_dtype, int64_t m, int64_t n, int64_t k,
                  q4_stream_t stream);

/* Bytes of workspace q4_gemm needs for this shape with fp16 activations (0
 * when none). */
size_t q4_gemm_workspace_size(int64_t m, int64_t n, int64_t k);

/* As q4_gemm_workspace_size for activations of dtype x_dtype (0 for fp32
 * activations, an unknown dtype or an invalid shape).  bf16 activations add
 * m * k * 2 bytes (rounded up to 256), where they are staged as fp16. */
size_t q4_gemm_workspace_size_dt(int64_t m, int64_t n, int64_t k, int x_dtype);

/* Prefill GEMM: y[m][n] = x[m][k] . dequant(packed)^T for any m >= 1 (the
 * page's GPU path onto matrix cores).  x is Q4_F32, Q4_F16 or Q4_BF16; y is
 * Q4_F32 or Q4_F16.
 *   - fp16 and bf16 activations: weight tiles are dequantised to fp16
 *     (w = (q - 8) * d rounded once) and contracted on fp16 matrix cores
 *     with fp32 accumulation; bf16 activations are first staged as fp16 in
 *     the workspace (round to nearest even).  Where that is not exact -- a
 *     block scale |d| > 8188, whose dequantised weights leave fp16's range,
 *     or a bf16 activation fp16 cannot hold -- the affected output tiles come
 *     out non-finite inside the kernel and are recomputed there on the exact
 *     route below, so every in-domain input gives a result within tolerance.
 *   - fp32 activations take the exact route for every tile: activations and
 *     dequantised weights in fp32 on fp32 matrix cores (several times slower
 *     than the fp16 tiles).
 * `workspace` must hold q4_gemm_workspace_size_dt(m, n, k, x_dtype) bytes (it
 * may be NULL when that is 0) and must not overlap x, y or packed; its
 * contents on entry are ignored.  A prompt processed in row chunks passes
 * x + c*rows*k and y + c*rows*n for chunk c. */
q4_status q4_gemm(const void *x, int x_dtype, const void *packed, void *y,
                  int y_dtype, int64_t m, int64_t n, int64_t k,
                  void *workspace, size_t workspace_bytes,
                  q4_stream_t stream);

/* Bytes of the fixed per-device scratch array behind q4_gemm_noalloc. */
#define Q4_NOALLOC_SCRATCH_BYTES (64u << 20)

/* q4_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, kernels and results as q4_gemm, with the workspace taken
 * from a fixed array of Q4_NOALLOC_SCRATCH_BYTES bytes that the library holds
 * on each device it runs on until the process ends.  The array is the current
 * device's (the device of `stream`); the first call on a device looks up its
 * address once.  Calls whose workspace need, q4_gemm_workspace_size_dt(m, n,
 * k, x_dtype), exceeds the array return Q4_ERR_SCRATCH before launching
 * anything.  The call itself allocates nothing.  Every call on one device
 * shares that device's array: calls that may overlap on one device (several
 * streams, several host threads) race on it and must be serialised by the
 * caller; its contents after a call are unspecified, and each call writes
 * every scratch byte it reads.  Arguments, errors and layouts are q4_gemm's. */
q4_status q4_gemm_noalloc(const void *x, int x_dtype, const void *packed, void *y,
                          int y_dtype, int64_t m, int64_t n, int64_t k,
                          q4_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBQ4_Q4_H */
