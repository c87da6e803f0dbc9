/*
 * kq_probe.h -- measurement instruments of libkq (gfx950): not part of the
 * product path.  They bound what the kernels of kq.h can reach on the same GPU
 * in the same session, the way the Bonsai page measures its matvec against a
 * streaming-read ceiling and a loads-only twin of the kernel ([BT] sec. 8.5,
 * "the matvec wall"): the twin issues exactly the GEMV's weight and
 * activation loads, with its grid and workgroup shape, and does nothing else;
 * an MFMA issue loop bounds the prefill GEMM the same way.
 *
 * Conventions as in kq.h: device pointers owned by the caller, asynchronous on
 * `stream` (a hipStream_t as void*, NULL = default stream), arguments checked
 * before any launch, no allocation, no synchronisation.
 */
#ifndef KQ_PROBE_H
#define KQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "kq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at `buf` (16-byte non-temporal loads,
 * XOR-reduced in registers; a workgroup writes its reduction to sink[0] only
 * when it equals 0x9E3779B9, so the loads cannot be dropped).  layout 0:
 * grid-stride over 16-byte units; layout 1: workgroup b reads the b-th of
 * `grid` contiguous chunks.  grid in 1..65536 workgroups of `block` threads
 * (64..1024, a multiple of 64).  bytes: a multiple of 16, at least 16.
 * sink: one device uint32.  Errors: KQ_EINVAL (NULL, bad layout), KQ_ESHAPE
 * (grid, block, bytes), KQ_EALIGN (buf or sink not 16-byte aligned),
 * KQ_EDEVICE. */
kq_status kq_probe_read(const void *buf, size_t bytes, int32_t layout,
                        int32_t grid, int32_t block, uint32_t *sink,
                        void *stream);

/* Matrix-core ceiling of the prefill GEMM's instruction: every wave of `grid`
 * workgroups of `block` threads issues `iters` rounds of 16 independent
 * v_mfma_f32_16x16x32_bf16 on operands held in registers, and nothing else
 * but one final sum of its accumulators (written to sink[0] only when its
 * bits equal 0x9E3779B9).  Floating-point operations per launch:
 * grid * (block / 64) * iters * 16 * 16384; the GEMM's rate is reported
 * against this reachable rate beside the datasheet peak, as the matvec is
 * reported against its streaming wall.  iters in 1..2^20, grid in 1..65536,
 * block in 64..1024 (a multiple of 64).  Errors: KQ_EINVAL (NULL sink),
 * KQ_ESHAPE, KQ_EALIGN (sink not 16-byte aligned), KQ_EDEVICE. */
kq_status kq_probe_mfma(int32_t iters, int32_t grid, int32_t block, uint32_t *sink,
                        void *stream);

/* Loads-only twin of kq_gemv(fmt, packed, N, K, x, M, block_len, NULL,
 * split_k, ...): the launch plan kq_gemv picks for these arguments (grid,
 * waves per workgroup, K slices), and per wave the same weight-code, scale
 * and activation loads at the same offsets with the same cache hints and the
 * same number of row blocks in flight -- without the rotation, the matrix
 * products or the reduction.  Writes sink[0] only as kq_probe_read does.
 * Errors: as kq_gemv (KQ_EUNSUPPORTED where kq_gemv has no plan). */
kq_status kq_probe_gemv_loads(kq_format fmt, const void *packed, int64_t N,
                              int64_t K, const float *x, int64_t M,
                              int32_t block_len, int32_t split_k,
                              uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KQ_PROBE_H */
