/*
 * libq4floor -- a plain streaming read of device memory on MI355X (gfx950).
 *
 * Measurement support for the decode GEMV's roofline, not part of the Q4_0
 * path: the batched decode stage of "Vertical disaggregation: maximizing
 * throughput on heterogeneous silicon" (section "Every cycle counts: custom
 * kernels") is bound by reading the packed weights, so the benchmark times
 * this kernel reading the same bytes, with no Q4_0 work, to show what one
 * launch streaming that many bytes costs on this part.
 */
#ifndef LIBQ4_READ_FLOOR_H
#define LIBQ4_READ_FLOOR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at device pointer `p` (16-byte aligned, bytes a multiple
 * of 16) once, as 16-byte loads spread over `workgroups` workgroups of 256
 * threads (grid-stride, four loads in flight per thread), and write each
 * thread's XOR of what it read to sink[workgroups * 256] (device memory the
 * caller owns; 4 bytes per thread), so no load can be dropped.  Asynchronous
 * on `stream` (a hipStream_t; NULL = the null stream).  Returns 0, 1 for an
 * invalid argument (NULL pointer, misalignment, workgroups < 1) or 5 when the
 * runtime refuses the launch.  Allocates nothing. */
int q4_read_floor(const void *p, size_t bytes, uint32_t *sink, int workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBQ4_READ_FLOOR_H */
