/*
 * libq4floor -- the matrix cores' sustained rate on MI355X (gfx950).
 *
 * Measurement support for the prefill GEMM's roofline, not part of the Q4_0
 * path.  The GEMM of "Vertical disaggregation: maximizing throughput on
 * heterogeneous silicon" (section "Every cycle counts: custom kernels") runs
 * on fp16 matrix products; under a long, dense load the chip lowers its
 * shader clock below the 2.4 GHz at which the quoted fp16 peak holds.  This
 * kernel does the GEMM's matrix-core work and nothing else -- no global
 * memory, no dequantisation, no barriers -- so the benchmark can time it
 * beside the GEMM and report what part of the attainable rate the GEMM
 * reaches.
 *
 * Work: each workgroup is 8 waves (two per SIMD, as the GEMM's 256 x 256
 * tile).  Per step every wave reads four A and two B operand fragments of
 * 8 halves per lane from LDS (the GEMM tile's fragment reads per 8 products)
 * and issues 8 v_mfma_f32_32x32x16_f16 into 4 x 2 fp32 accumulator tiles.
 * The LDS holds 32768 fp16 values h[i] drawn from `seed` (below); step s
 * reads the 4096 halves starting at 4096 (s % 8): lane l's A fragment i is
 * halves 512 i + 8 l .. + 7 of that window and its B fragment j is halves
 * 2048 + 512 j + 8 l .. + 7 (every wave reads the same fragments).
 * Value i: z = mix(i * 0x9E3779B1 ^ seed) with mix(z) = z ^= z >> 15,
 * z *= 0x2C1B3C6D, z ^= z >> 12, z *= 0x297A2D39, z ^= z >> 15 (32-bit
 * wrap-around arithmetic); the half's bits are (z & 0x8000) |
 * ((14 + ((z >> 10) & 1)) << 10) | (z & 0x3FF): random signs and mantissas
 * with magnitudes in [0.5, 2), as toggling as real operands.
 * Flops per launch: workgroups * 8 * iters * 8 * 2 * 32 * 32 * 16.
 */
#ifndef LIBQ4_MFMA_CEILING_H
#define LIBQ4_MFMA_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Run `iters` steps on `workgroups` workgroups of 512 threads and write each
 * thread's sum of its 128 accumulator values to sink[workgroups * 512]
 * (device memory the caller owns; 4 bytes per thread), so no product can be
 * dropped.  Asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 * Returns 0, 1 for an invalid argument (NULL sink, workgroups < 1,
 * iters < 1) or 5 when the runtime refuses the launch.  Allocates nothing. */
int q4_mfma_ceiling(uint32_t seed, int iters, float *sink, int workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBQ4_MFMA_CEILING_H */
