/*
 * kq.h -- quantized-weight GEMV / GEMM for AMD MI355X (gfx950): the C ABI.
 *
 * What is computed (the pages this library follows):
 *   [BT] "Bonsai 2 27B -- ternary g128 + blockwise Hadamard: the packing
 *        contract for a Core AI port" (Core AI model zoo knowledge page)
 *        sec. 3.1  PQ2_0 block, quantizer d = max|w|, q = round(w/d) + 1,
 *                  code q -> (q-1)*d, and the "word view" of the codes;
 *        sec. 3.2  PTQ1_0, the same trits in base-3 bytes (load-time
 *                  transcode to PQ2_0);
 *        sec. 4.1  R = (1/sqrt(n)) H_n S, Sylvester natural order,
 *                  applied block-diagonally along K;
 *        sec. 4.2  runtime order of a folded linear: sign flip, blockwise
 *                  transform, then the ternary product y = W' (R x).
 *   [KA] "Kipp architecture" page, "Weight quantization": Q8_0, 32-weight
 *        blocks with one fp16 scale, quantized against the fp16-rounded
 *        scale; decode kernels for one token, tiled matrix kernels for
 *        prompts.
 *   [KB] "Kipp Benchmarks" page: Q8_0 dequantization d*q; the dequantize-
 *        once-per-tile prefill kernels ("Quantized projections on the
 *        tensor units").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer owned by the caller
 *   (for example PyTorch tensors).  The library never allocates, frees,
 *   copies to or from the host, or synchronises; it only enqueues kernels on
 *   `stream` (a hipStream_t passed as void*; NULL is the default stream) and
 *   returns.  Results are ready when the stream reaches that point.
 * Layouts.  Row-major, last index contiguous:  W [N][K],  x and x' [M][K],
 *   y [M][N].  N counts output rows, K is the reduction (the page's "ne
 *   order, K first").
 * Packed weights (planar device layout).  kq_packed_bytes(fmt, N, K) bytes:
 *     qs plane : the 32 code bytes of every block (nb blocks per row:
 *                K/128 for PQ2_0, K/32 for Q8_0), in tiles of 16 rows x
 *                one block: tile (t, b) holds block b of rows 16t..16t+15
 *                and starts at byte 512 * (t * nb + b); inside it, row
 *                n % 16 occupies bytes 32 * (n % 16) .. +31.  Rows past N
 *                in the last tile are zero.  Plane size:
 *                ceil(N/16) * 16 * nb * 32 bytes.  Inside a block: for
 *                Q8_0 the 32 int8 codes in order; for PQ2_0, 8 little-endian
 *                u32 words, word i holding the codes of elements 16*i + j
 *                (j = 0..15) -- the block's word view ([BT] 3.1 "Word
 *                view": code j at bits 2*j, 2*j + 1) with the high bit of
 *                each code moved: bit 0 of code j at bit 2*j, bit 1 at bit
 *                (2*j + 3) mod 32 (the odd bits rotated up by two).
 *     d plane  : at byte offset round_up(qs plane size, 256): one IEEE
 *                binary16 scale per block (little endian), in chunks of
 *                16 rows x 8 blocks: the scale of block b of row n sits in
 *                chunk (n / 16, b / 8), which starts at byte
 *                256 * ((n / 16) * C + b / 8), C = ceil(nb / 8), at byte
 *                16 * (n % 16) + 2 * (b % 8) within it.  Slots of rows past N
 *                and of blocks past nb are zero.  Plane size:
 *                ceil(N/16) * C * 256 bytes.
 *   This is a lossless re-arrangement of the GGUF-style array of 34-byte
 *   blocks { fp16 d; uint8 qs[32] }: the scales move out, the code blocks of
 *   16 rows are interleaved so that a wave's 16 rows x 2 blocks are one
 *   contiguous KiB, and a row's scales for 8 consecutive blocks are 16
 *   contiguous bytes next to those of the other 15 rows of its tile.
 * Alignment.  All pointers must be 16-byte aligned, else KQ_EALIGN.
 * Errors.  Arguments are validated before anything is enqueued; on any
 *   error nothing is launched and no output byte is written.  A failed
 *   launch returns KQ_EDEVICE.  No HIP type or HIP error code crosses this
 *   interface.  Contents of device memory (finite weights, sign values)
 *   are preconditions: the library cannot read them without a sync.
 * Threads.  No global mutable state; calls on different streams may run
 *   concurrently.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KQ_FMT_PQ2_0 = 1, /* 128 weights: fp16 d + 32 B of 2-bit codes (34 B) */
    KQ_FMT_Q8_0 = 2   /* 32 weights: fp16 d + 32 int8 (34 B)              */
} kq_format;

typedef enum {
    KQ_F32 = 0,  /* IEEE binary32 */
    KQ_BF16 = 1  /* bfloat16 (upper half of a binary32) */
} kq_dtype;

typedef enum {
    KQ_OK = 0,
    KQ_EINVAL = 1,       /* NULL pointer, unknown enum, negative size      */
    KQ_ESHAPE = 2,       /* K, N, M, block_len or split_k out of contract  */
    KQ_EALIGN = 3,       /* a pointer is not 16-byte aligned               */
    KQ_EWORKSPACE = 4,   /* workspace missing or smaller than required     */
    KQ_EUNSUPPORTED = 5, /* valid but unsupported combination              */
    KQ_EDEVICE = 6       /* the HIP runtime rejected a launch              */
} kq_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *kq_status_string(kq_status s);

/* Bytes of the planar packed buffer for an N x K matrix in `fmt`, or 0 if
 * the shape is invalid (K % 128 for PQ2_0, K % 32 for Q8_0, N >= 1). */
size_t kq_packed_bytes(kq_format fmt, int64_t N, int64_t K);

/* PQ2_0 quantizer, [BT] 3.1.  For every row n and 128-group of W [N][K]
 * (fp32): d16 = fp16_rne(max|w|), and for each weight
 * q = round_half_away(w / f32(d16)) + 1 in {0,1,2} with IEEE fp32 division
 * (q = 1 for every weight of a group whose d16 is 0).  Writes the planar
 * buffer `packed` (kq_packed_bytes(KQ_FMT_PQ2_0, N, K) bytes); the bytes
 * are deterministic.  Precondition: W finite with max|w| < 65520 per group.
 * Errors: KQ_EINVAL (NULL), KQ_ESHAPE (N < 1, K < 128, K % 128),
 * KQ_EALIGN. */
kq_status kq_pack_pq2(const float *W, int64_t N, int64_t K, void *packed,
                      void *stream);

/* Q8_0 quantizer, [KA].  Per 32-group: d32 = max|w| / 127 (fp32 division),
 * d16 = fp16_rne(d32); q = round_half_away(w / f32(d16)) clamped to
 * [-127, 127] (q = 0 when d16 is 0).  Writes the planar buffer.
 * Errors as kq_pack_pq2, with K % 32. */
kq_status kq_pack_q8(const float *W, int64_t N, int64_t K, void *packed,
                     void *stream);

/* PTQ1_0 -> PQ2_0 at load time, [BT] 3.2: PTQ1_0 carries the same trits
 * (code values 0, 1, 2) and fp16 scales as PQ2_0 at 1.75 bits per weight, so
 * it is a download format that is transcoded losslessly once and then used
 * through the PQ2_0 entry points.  ptq1: N * K/128 blocks of 28 bytes, row
 * after row, block after block along K; each block is 24 bytes of five
 * base-3 digits and 2 bytes of four, then the fp16 scale (little endian,
 * last).  Element e of a block is digit e/16 of byte e%16 (e < 80), digit
 * (e-80)/8 of byte 16 + (e-80)%8 (e < 120), or digit (e-120)/2 of byte
 * 24 + (e-120)%2; digit n of byte q is ((q * 3^n) mod 256) * 3 / 256, the
 * first digit most significant.  Every byte value decodes.  Writes the planar
 * PQ2_0 buffer `packed` (kq_packed_bytes(KQ_FMT_PQ2_0, N, K) bytes) exactly as
 * kq_pack_pq2 would lay out the same codes and scales.
 * Errors: KQ_EINVAL (NULL, negative size), KQ_ESHAPE (N < 1, K < 128,
 * K % 128), KQ_EALIGN. */
kq_status kq_transcode_ptq1(const void *ptq1, int64_t N, int64_t K,
                            void *packed, void *stream);

/* Dequantize a planar buffer to fp32 W_out [N][K]: (q-1)*d for PQ2_0 (a
 * foreign code 3 decodes to 2*d), d*q for Q8_0 ([BT] 3.1, [KB]).  Exact.
 * Errors: KQ_EINVAL, KQ_ESHAPE, KQ_EALIGN. */
kq_status kq_unpack(kq_format fmt, const void *packed, int64_t N, int64_t K,
                    float *W_out, void *stream);

/* Blockwise rotation x' = (1/sqrt(n)) H_n (s (.) x) of every n-block of
 * every row of x [M][K], [BT] 4.1-4.2 (sign first, then the transform; H_n
 * Sylvester natural order).  n = block_len in {1, 2, 4, ..., 1024}, n | K,
 * and K % 16 == 0.  signs: K int8 entries (negative -> -1, else +1) or NULL
 * for all +1.  x_dt / xr_dt: KQ_F32 or KQ_BF16 (arithmetic in fp32, one
 * round-to-nearest-even to bf16 at the store when xr_dt is KQ_BF16).  x and
 * xr may not overlap.  Errors: KQ_EINVAL, KQ_ESHAPE, KQ_EALIGN. */
kq_status kq_hadamard_blocks(const void *x, kq_dtype x_dt, void *xr,
                             kq_dtype xr_dt, int64_t M, int64_t K,
                             int32_t block_len, const int8_t *signs,
                             void *stream);

/* Workspace bytes kq_gemv (op = 0) or kq_gemm (op = 1) needs for these
 * arguments; 0 means none.  split_k as for kq_gemv (0 = automatic). */
size_t kq_workspace_bytes(int32_t op, kq_format fmt, int64_t M, int64_t N,
                          int64_t K, int32_t block_len, int32_t split_k);

/* Quantized GEMV for M in 1..8 activation rows (one decode step, or a few
 * sequences sharing the weights).  The folded linear of [BT] 4.2 (sign flip,
 * blockwise transform, then the ternary matvec y = W' (R x)), with the
 * PQ2_0 decode of [BT] 3.1 or the Q8_0 decode d*q of [KA] "Weight
 * quantization" / [KB] (one decode kernel per token, reading every weight
 * once for all M rows):
 *     y[m][n] = sum_k deq(W)[n][k] * x'[m][k],   x' = rotation of x
 * with deq as in kq_unpack and x' as in kq_hadamard_blocks (block_len 0:
 * x' = x (.) s, no transform), except that a PQ2_0 code 3, which is not a
 * value of the format (only codes 0, 1, 2 are), counts as a zero weight here
 * (kq_unpack and kq_gemm read it as 2*d).  x is fp32 [M][K]; y is fp32
 * [M][N].
 * Arithmetic: x' in fp32, codes decoded exactly, fp32 accumulation; each
 * output is within 1e-3 * sum_k |deq(W)[n][k] x'[m][k]| of the exact value.
 * Representation limits: PQ2_0 carries each x' element as four e5m2 terms
 * (to 2^-12 of itself, down to about 2^-30 of the largest |x'| in its
 * 128-group), and the matrix core adds the 128 products of a group aligned to
 * the largest of them, keeping about 17 bits below it; a group whose largest
 * |w x'| dwarfs the rest can therefore lose up to about 2^-10 of that
 * product (measured: 7.7e-4 of the bound for an element 2^24 times the others
 * with no rotation; near 1e-6 of it with a 128-element rotation, which spreads
 * such elements over the block).  Q8_0 with M <= 4 holds each element to
 * 2^-30 of the largest |x'| of its row within the K slice (an output whose
 * weights touch only elements more than about 10^6 below that can miss the
 * bound); M >= 5: 2^-17 of itself.
 * split_k: 1 = one pass over K; S > 1 splits K into S contiguous ranges of
 * whole blocks whose fp32 partial sums are added in ascending order
 * (deterministic, no atomics); 0 = chosen by the library.  Results are
 * bitwise reproducible for a given (split_k, M, N, K).
 * workspace: at least kq_workspace_bytes(0, ...) bytes of device memory
 * (the split partials), or NULL when that is 0.
 * Errors: KQ_EINVAL, KQ_ESHAPE (M not in 1..8, N < 1, K not a multiple of
 * the block, bad block_len, split_k < 0 or larger than K's block count),
 * KQ_EALIGN, KQ_EWORKSPACE, KQ_EDEVICE; KQ_EUNSUPPORTED when no launch plan
 * fits: more K slices than rotation blocks, a K slice too wide for one
 * workgroup's LDS, more than 512 MiB of packed codes per workgroup (a
 * workgroup streams about 1/256 of the rows), or N of 2^31 - 32 rows or
 * more. */
kq_status kq_gemv(kq_format fmt, const void *packed, int64_t N, int64_t K,
                  const float *x, int64_t M, int32_t block_len,
                  const int8_t *signs, int32_t split_k, float *y,
                  void *workspace, size_t ws_bytes, void *stream);

/* kq_gemv for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same arguments
 * without workspace, the same kernels and bitwise the same results.  The
 * split-K partials, the only scratch memory kq_gemv uses, go to a static
 * device array of the library, 8 MiB per GPU (S * M * N * 4 bytes at most,
 * S the split kq_gemv would use; larger plans are rejected with
 * KQ_EWORKSPACE), held by every GPU the library runs on until the process
 * ends.  No allocation, no free, no synchronisation.  The array's address is
 * resolved on the first call on each device, with the caller's device
 * current (the stream must belong to it).  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams, threads)
 * race and must be serialised by the caller; the array keeps the last call's
 * partials, and nothing needs it to start at zero.
 * Errors: as kq_gemv (KQ_EWORKSPACE: the plan needs more than 8 MiB;
 * KQ_EDEVICE: the runtime could not give the array's address). */
kq_status kq_gemv_noalloc(kq_format fmt, const void *packed, int64_t N,
                          int64_t K, const float *x, int64_t M,
                          int32_t block_len, const int8_t *signs,
                          int32_t split_k, float *y, void *stream);

/* Several weight sets times one activation in one launch: for s < nsets,
 *     y[s][m][n] = sum_k deq(W_s)[n][k] * x'[m][k]
 * with every W_s an N[s] x K matrix in `fmt` and x' as in kq_gemv (shared:
 * rotated once per workgroup), so projections fed by the same activation
 * (q, k and v; gate and up) take a single launch ([BT] sec. 8.7, the matvec
 * over several weight sets).  packed, N and y are HOST
 * arrays of nsets entries; packed[s] and y[s] are device pointers (planar
 * buffer of kq_packed_bytes(fmt, N[s], K) bytes; fp32 [M][N[s]]).  One pass
 * over K (no split, no workspace).  Each y[s] is bit-identical to
 * kq_gemv(fmt, packed[s], N[s], K, x, M, block_len, signs, 1, y[s], ...):
 * same arithmetic, same fixed reduction order.  The outputs may not overlap
 * each other or x.
 * Errors: KQ_EINVAL (NULL array or entry, negative size), KQ_ESHAPE (nsets
 * not in 1..4, or as kq_gemv for any set), KQ_EALIGN, KQ_EUNSUPPORTED (no
 * one-slice plan: the K slice does not fit one workgroup's LDS, or more than
 * 512 MiB of codes per workgroup), KQ_EDEVICE. */
kq_status kq_gemv_multi(kq_format fmt, int32_t nsets, const void *const *packed,
                        const int64_t *N, int64_t K, const float *x, int64_t M,
                        int32_t block_len, const int8_t *signs, float *const *y,
                        void *stream);

/* Prefill GEMM (many tokens), dequantize-once-per-tile ([KB] "Quantized
 * projections on the tensor units": each weight block becomes a bf16 tile
 * once, then the matrix units; [BT] 8.3, the chunked prefill's tiled GEMM):
 *     y[m][n] = sum_k bf16(deq(W)[n][k]) * bf16(x'[m][k])   (fp32 accumulate)
 * with deq as in kq_unpack, for PQ2_0 or Q8_0 weights.  x is [M][K] in x_dt
 * (KQ_BF16 or KQ_F32); x' (as in kq_hadamard_blocks) is rounded once to
 * bf16; y is fp32 [M][N].  Each output is within 1e-2 * sum_k |deq(W) x'| of
 * the exact value.  M >= 1, N >= 1, K a multiple of the block (128 or 32).
 * The token tile follows M: 16 tokens up to M = 16, 64 up to M = 96, else
 * 256 (a 16- or 64-token chunk does not pay for a 256-row tile).  With the
 * 16- and 64-token tiles K is split into slices (about 1024 workgroups in
 * all), whose fp32 partial products are added in slice order: the result is
 * bitwise reproducible for a given (M, N, K).
 * workspace: at least kq_workspace_bytes(1, ...) bytes (room for the bf16 x',
 * then the slices' fp32 partials [S][M][N]); needed when x' is staged
 * (block_len > 0, signs, or fp32 x) or K is split (the 16- and 64-token tiles
 * when there are fewer than 1024 output tiles), else it may be NULL.
 * Errors: as kq_gemv; KQ_EUNSUPPORTED for K > 2^21 (32-bit buffer ranges of
 * a 256-row activation tile) or more than 2^31 - 1 output tiles. */
kq_status kq_gemm(kq_format fmt, const void *packed, int64_t N, int64_t K,
                  const void *x, kq_dtype x_dt, int64_t M, int32_t block_len,
                  const int8_t *signs, float *y, void *workspace,
                  size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KQ_H */
