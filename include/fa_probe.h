/*
 * fa_probe.h -- measurement probes of libfa.so.  Not part of the
 * computational ABI in fa.h: kernels that measure, on the GPU at hand, the
 * rate of the bare operation each attention kernel is bound by -- a stream of
 * bf16 matrix-core products for the prefill, a streaming HBM read for the
 * split-KV decode, a streaming copy for the row softmax -- so that a
 * benchmark can report its kernels against these measured ceilings beside the
 * published peaks.  All run asynchronously on `stream` (a hipStream_t, NULL
 * for the default stream) and allocate nothing.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core stream: `blocks` workgroups of 256 threads (4 waves each); every
 * wave issues `iters` rounds of eight v_mfma_f32_32x32x16_bf16 products into
 * four independent accumulator chains, on pseudo-random bf16 operands held in
 * registers (a different operand pair for each product of a round; no memory
 * traffic in the loop).  Executed bf16 FLOPs per call =
 * blocks * 4 * iters * 8 * 32768.  Each thread writes the sum of its
 * accumulators to sink[256 * block + thread] (device, fp32, 256 * blocks
 * entries, caller-owned); the sums grow linearly with iters.
 * Errors: FA_ERR_INVALID_ARG for a NULL sink, blocks < 1 or iters < 1;
 * FA_ERR_HIP if the launch fails.
 */
fa_status fa_probe_mfma(float *sink, int blocks, int iters, void *stream);

/*
 * Streaming read: `blocks` workgroups of 256 threads read the `bytes` bytes at
 * src (device, 16-byte aligned, bytes a multiple of 16) once, in 16-byte
 * nontemporal loads, each workgroup one contiguous run of 64 KiB chunks
 * (consecutive workgroups, consecutive runs), and each thread writes the XOR of
 * the 32-bit words it read to sink[256 * block + thread] (device, uint32,
 * 256 * blocks entries, caller-owned): the XOR of all of sink is the XOR of
 * every 32-bit word of the buffer.  bytes = 0 (src may then be NULL) writes
 * zeros.
 * Errors: FA_ERR_INVALID_ARG for a NULL sink, blocks < 1, bytes not a multiple
 * of 16, or (bytes > 0) a NULL or misaligned src; FA_ERR_HIP if the launch
 * fails.
 */
fa_status fa_probe_read(const void *src, size_t bytes, uint32_t *sink, int blocks, void *stream);

/*
 * Streaming copy: `blocks` workgroups of 256 threads copy the `bytes` bytes at
 * src to dst (both device, 16-byte aligned, the two ranges disjoint, bytes a
 * multiple of 16) once, in 16-byte nontemporal loads and stores, each
 * workgroup one contiguous run of 64 KiB chunks as in the streaming read: the
 * traffic of a kernel that reads an array once and writes one of the same
 * size.  bytes = 0 does nothing (src and dst may then be NULL).
 * Errors: FA_ERR_INVALID_ARG for blocks < 1, bytes not a multiple of 16, or
 * (bytes > 0) a NULL or misaligned src or dst, or ranges that overlap;
 * FA_ERR_HIP if the launch fails.
 */
fa_status fa_probe_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
