/*
 * kq_oracle.h -- the CPU oracle for the quantized GEMV / GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and kq_oracle.c are a plain, slow,
 * deliberately obvious CPU implementation of what the GPU path computes.  Only
 * the test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no code, header, table or constant with the HIP library
 * (gemm_kq_gemv_amd/csrc), and neither side includes the other.
 *
 * Sources (the web pages this project follows):
 *   [BT]  "Bonsai 2 27B -- ternary g128 + blockwise Hadamard: the packing
 *         contract for a Core AI port" (Core AI model zoo knowledge page):
 *         sec. 3.1 (PQ2_0 block, quantizer, word view), sec. 3.2 (PTQ1_0
 *         trit block and its element order), sec. 4.1 (rotation
 *         definition, blockwise application), sec. 4.2 (runtime order).
 *   [KA]  "Kipp architecture" page: "Weight quantization" (Q8_0: 32-weight
 *         blocks, fp16 scale, quantized against the fp16-rounded scale).
 *   [KB]  "Kipp Benchmarks" page: Q8_0 decode is d*q; the 136-byte
 *         128-value row (4 x 34 B) that fixes the 34-byte Q8_0 block.
 *   [JL]  "jitllm -- the scoreboard": section "AND THEN THE PACKER WAS
 *         GENERATED" (round half away from zero; zero window masked).
 *
 * Precision: every product and rotation is carried in IEEE binary64.  The
 * quantizers follow the pages' fp32 arithmetic (fp32 amax, fp32 division by
 * the fp16-rounded scale) because the packed bytes are defined by it.
 *
 * Parity pins: every function below is pinned by tests that do not re-type
 * its own formula (exhaustive codec checks against NumPy, hand-derived
 * fixtures, Hadamard identities checked against SciPy, closed forms and
 * brute force).  No function here is "parity unpinned".
 */
#ifndef KQ_ORACLE_H
#define KQ_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar codecs (IEEE 754 binary16 / bfloat16, round to nearest even) */
uint16_t kqo_f16_from_f32(float f);
float    kqo_f32_from_f16(uint16_t h);
uint16_t kqo_bf16_from_f32(float f);
float    kqo_f32_from_bf16(uint16_t b);
/* bulk versions over n elements, for exhaustive tests */
void kqo_f16_from_f32_n(const float *in, uint16_t *out, int64_t n);
void kqo_f32_from_f16_n(const uint16_t *in, float *out, int64_t n);
void kqo_bf16_from_f32_n(const float *in, uint16_t *out, int64_t n);
void kqo_f32_from_bf16_n(const uint16_t *in, float *out, int64_t n);

/* ---- block formats ------------------------------------------------------
 * PQ2_0 [BT 3.1]: 128 weights -> { fp16 d (little endian); uint8 qs[32] },
 *   34 bytes.  Element j sits in byte j/4 at bit offset 2*(j%4); code q in
 *   {0,1,2} decodes to (q-1)*d.
 * Q8_0  [KA, KB]: 32 weights -> { fp16 d; int8 qs[32] }, 34 bytes; decodes
 *   to d*q.
 * W is row-major [N][K] (K contiguous); each row is split into K/128 (PQ2_0)
 * or K/32 (Q8_0) consecutive blocks.  The AoS stream is row after row, block
 * after block.  Return 0 on success, -1 on a bad shape.
 */
int kqo_pack_pq2_aos(const float *W, int64_t N, int64_t K, uint8_t *aos);
int kqo_pack_q8_aos(const float *W, int64_t N, int64_t K, uint8_t *aos);

/* Planar ("split") device layout of the library, restated independently:
 * the 32 code bytes of each block, grouped in tiles of 16 rows x one block
 * (512 bytes; row r of the tile at byte 32*r), tiles ordered by 16-row block
 * and then by block along K, the last tile zero-padded past row N; then, at
 * the first 256-byte boundary after them, the fp16 scales in chunks of 16
 * rows x 8 blocks (256 bytes; row r at byte 16*r, block b%8 at 2*(b%8)),
 * chunks ordered by 16-row block and then by 8-block run along K, slots past
 * N or past the row's blocks zero.  [BT 3.1 "Word view"]: the code bytes of a
 * block are a reinterpretation of its qs bytes; only their place moves.
 * fmt: 1 = PQ2_0, 2 = Q8_0. */
int64_t kqo_planar_bytes(int fmt, int64_t N, int64_t K);
int kqo_aos_to_planar(int fmt, const uint8_t *aos, int64_t N, int64_t K,
                      uint8_t *planar);

/* Decoders.  Byte view per [BT 3.1]: element j of a block from byte j/4,
 * bits 2*(j%4).  Code 3 (never produced) decodes as (3-1)*d.  Output in
 * binary64 ([N][K]).  The word-view decoder reads each 4-byte group as a
 * little-endian u32 and takes element 16*i+j from bits 2*j of word i -- an
 * independent reading of the same bytes that the page states is identical. */
int kqo_unpack_pq2_aos(const uint8_t *aos, int64_t N, int64_t K, double *W);
int kqo_unpack_pq2_aos_words(const uint8_t *aos, int64_t N, int64_t K, double *W);
int kqo_unpack_q8_aos(const uint8_t *aos, int64_t N, int64_t K, double *W);

/* ---- PTQ1_0 [BT 3.2] ----------------------------------------------------
 * 128 trits t in {0,1,2} (the PQ2_0 code values, (t-1)*d) per block: 24 bytes
 * of five trits (elements 0..79: element 16n + m is trit n of byte m; 80..119:
 * element 80 + 8n + m is trit n of byte 16 + m), 2 bytes of four trits
 * (element 120 + 2n + h is trit n of byte 24 + h), then fp16 d (little
 * endian, last): 28 bytes.  A byte of trits t0..t4 (t0 most significant) is
 * ceil(256 (81 t0 + 27 t1 + 9 t2 + 3 t3 + t4) / 243), a four-trit byte read
 * as t4 = 0; trit n of byte q is ((q 3^n) mod 256) * 3 / 256 rounded down.
 * pq2_to_ptq1: -1 if a PQ2_0 block holds code 3 (not a trit).  ptq1_to_pq2
 * is the lossless transcode to PQ2_0 blocks that [BT 3.2] recommends at load
 * time; every byte value decodes (to trits 0..2). */
int kqo_pq2_to_ptq1_aos(const uint8_t *pq2, int64_t N, int64_t K, uint8_t *ptq1);
int kqo_ptq1_to_pq2_aos(const uint8_t *ptq1, int64_t N, int64_t K, uint8_t *pq2);
int kqo_unpack_ptq1_aos(const uint8_t *ptq1, int64_t N, int64_t K, double *W);

/* ---- rotation [BT 4.1, 4.2] --------------------------------------------
 * H_n[r][c] = (-1)^popcount(r & c)  (Sylvester, natural order), n = 2^i.
 * kqo_hadamard_matrix writes the n*n entries as int8 (+1/-1). */
int kqo_hadamard_matrix(int32_t n, int8_t *H);
/* x' = (1/sqrt(n)) * H_n * (s (.) x) applied to each n-block of every row of
 * x [M][K], in binary64 with an explicit matrix product.  signs: K entries,
 * negative means -1, otherwise +1; NULL means all +1.  n == 0: x' = x * s
 * (no transform).  Returns -1 if n is not 0 or a power of two <= 1024, or
 * n does not divide K. */
int kqo_rotate(const double *x, int64_t M, int64_t K, int32_t n,
               const int8_t *signs, double *xr);

/* ---- product -------------------------------------------------------------
 * y[m][n]   = sum_k W[n][k] * xr[m][k]           (binary64)
 * bnd[m][n] = sum_k |W[n][k] * xr[m][k]|          (the per-row error scale)
 * Rows n are distributed over OpenMP threads; each dot product is a plain
 * ascending-k loop. bnd may be NULL. */
void kqo_matmul(const double *W, const double *xr, int64_t M, int64_t N,
                int64_t K, double *y, double *bnd);

/* ---- whole path, composed of the steps above (CPU baseline leg) ----------
 * y = unpack(aos) * rotate(x) for fmt 1 (PQ2_0) or 2 (Q8_0); x is fp32
 * [M][K]; y and bnd are binary64 [M][N].  Returns -1 on bad arguments. */
int kqo_gemv_aos(int fmt, const uint8_t *aos, int64_t N, int64_t K,
                 const float *x, int64_t M, int32_t block_len,
                 const int8_t *signs, double *y, double *bnd);

/* number of OpenMP threads kqo_matmul uses; set it (n >= 1) */
int kqo_num_threads(void);
void kqo_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif /* KQ_ORACLE_H */
