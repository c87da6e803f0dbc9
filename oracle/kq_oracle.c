/*
 * kq_oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see kq_oracle.h).
 *
 * Written to be checked by eye against the pages:
 *   [BT] Bonsai 2 27B ternary g128 + blockwise Hadamard page, sec. 3.1, 4.1, 4.2
 *   [KA] Kipp architecture page, "Weight quantization"
 *   [KB] Kipp Benchmarks page (Q8_0 dequant d*q; 34-byte block)
 *   [JL] jitllm scoreboard, "AND THEN THE PACKER WAS GENERATED"
 * Build: gcc -O2 -std=c11 -fopenmp -fPIC -shared (no -ffast-math: every fp32
 * division below must be the IEEE correctly rounded one).
 */
#include "kq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ======================================================================== */
/* IEEE 754 binary16 and bfloat16, written from the encoding definitions.   */
/* ======================================================================== */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Round-to-nearest-even of the integer m / 2^shift (shift >= 1). */
static uint32_t rne_shift(uint32_t m, int shift)
{
    uint32_t q = m >> shift;
    uint32_t rem = m & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;
    return q;
}

uint16_t kqo_f16_from_f32(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t ef = (u >> 23) & 0xFFu;      /* binary32 biased exponent */
    uint32_t mf = u & 0x7FFFFFu;          /* binary32 fraction */

    if (ef == 0xFFu) {                    /* Inf or NaN */
        if (mf == 0) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | 0x7E00u | (mf >> 13)); /* quiet NaN */
    }
    if (ef == 0)                          /* zero or binary32 subnormal: */
        return sign;                      /* |f| < 2^-126, far below 2^-25 */

    /* |f| = m * 2^(ef-150) with m the 24-bit significand. */
    uint32_t m = mf | 0x800000u;
    int e16 = (int)ef - 127 + 15;         /* binary16 biased exponent */

    if (e16 <= 0) {
        /* binary16 subnormal range: result is round(|f| / 2^-24) units of
         * 2^-24, i.e. m * 2^(ef-126). */
        int shift = 126 - (int)ef;        /* >= 14 here */
        if (shift > 24)                   /* |f| < 2^-25 (or == 2^-25: tie to 0) */
            return sign;
        uint32_t q = rne_shift(m, shift); /* may carry to 0x400 = min normal */
        return (uint16_t)(sign | q);
    }
    uint32_t q = rne_shift(m, 13);        /* 11-bit significand, rounded */
    if (q == 0x800u) { q = 0x400u; e16 += 1; }
    if (e16 >= 31) return (uint16_t)(sign | 0x7C00u); /* overflow to Inf */
    return (uint16_t)(sign | ((uint32_t)e16 << 10) | (q & 0x3FFu));
}

float kqo_f32_from_f16(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = ((uint32_t)h >> 10) & 0x1Fu;
    uint32_t m = (uint32_t)h & 0x3FFu;
    if (e == 0x1Fu)                       /* Inf / NaN (NaN stays quiet-able) */
        return bits_f32(sign | 0x7F800000u | (m << 13));
    if (e == 0) {                         /* zero or subnormal: m * 2^-24 */
        float v = (float)m * 0x1p-24f;    /* exact: m < 2^10 */
        return sign ? -v : v;
    }
    return bits_f32(sign | ((e - 15u + 127u) << 23) | (m << 13));
}

uint16_t kqo_bf16_from_f32(float f)
{
    uint32_t u = f32_bits(f);
    if (((u >> 23) & 0xFFu) == 0xFFu && (u & 0x7FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);           /* quiet NaN */
    /* keep the top 16 bits, round on the low 16 (ties to even); a carry out
     * of the fraction correctly bumps the exponent, up to Inf */
    uint32_t q = rne_shift(u & 0x7FFFFFFFu, 16);
    return (uint16_t)(((u >> 16) & 0x8000u) | q);
}

float kqo_f32_from_bf16(uint16_t b) { return bits_f32((uint32_t)b << 16); }

void kqo_f16_from_f32_n(const float *in, uint16_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = kqo_f16_from_f32(in[i]); }
void kqo_f32_from_f16_n(const uint16_t *in, float *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = kqo_f32_from_f16(in[i]); }
void kqo_bf16_from_f32_n(const float *in, uint16_t *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = kqo_bf16_from_f32(in[i]); }
void kqo_f32_from_bf16_n(const uint16_t *in, float *out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = kqo_f32_from_bf16(in[i]); }

/* ======================================================================== */
/* Quantizers.                                                              */
/* ======================================================================== */

/* C roundf: nearest integer, halfway cases away from zero [JL]. */
static int round_half_away(float r) { return (int)roundf(r); }

static float block_amax(const float *w, int len)
{
    float a = 0.0f;
    for (int j = 0; j < len; ++j) {
        float v = fabsf(w[j]);
        if (v > a) a = v;
    }
    return a;
}

/* [BT 3.1]: d = max|w| over the 128-group; q = round(w/d) + 1; element j in
 * byte j/4 at bit offset 2*(j%4).  d is stored as fp16, and the codes are
 * computed against that stored (fp16-rounded) value so that encoder and
 * decoder agree exactly ([KA] "Weight quantization").  An all-zero block has
 * d = 0 and every code 1 (the zero window is masked, [JL]). */
int kqo_pack_pq2_aos(const float *W, int64_t N, int64_t K, uint8_t *aos)
{
    if (N < 0 || K <= 0 || K % 128) return -1;
    int64_t nb = K / 128;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *w = W + n * K + b * 128;
            uint8_t *blk = aos + (n * nb + b) * 34;
            uint16_t d16 = kqo_f16_from_f32(block_amax(w, 128));
            float dF = kqo_f32_from_f16(d16);
            blk[0] = (uint8_t)(d16 & 0xFF);       /* little-endian fp16 */
            blk[1] = (uint8_t)(d16 >> 8);
            uint8_t *qs = blk + 2;
            memset(qs, 0, 32);
            for (int j = 0; j < 128; ++j) {
                int q;
                if (dF == 0.0f) {
                    q = 1;
                } else {
                    float r = w[j] / dF;             /* IEEE fp32 division */
                    q = round_half_away(r) + 1;
                    if (q < 0) q = 0;                /* never taken for finite w */
                    if (q > 2) q = 2;
                }
                qs[j / 4] |= (uint8_t)(q << (2 * (j % 4)));
            }
        }
    }
    return 0;
}

/* Q8_0: 32-weight blocks; scale = max|w|/127 in fp32, rounded to fp16; each
 * weight is round(w / scale) against the fp16-rounded scale ([KA]), ties away
 * from zero ([JL]); block = { fp16 d; int8 q[32] } (34 bytes, [KB]). */
int kqo_pack_q8_aos(const float *W, int64_t N, int64_t K, uint8_t *aos)
{
    if (N < 0 || K <= 0 || K % 32) return -1;
    int64_t nb = K / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *w = W + n * K + b * 32;
            uint8_t *blk = aos + (n * nb + b) * 34;
            float d32 = block_amax(w, 32) / 127.0f;  /* IEEE fp32 division */
            uint16_t d16 = kqo_f16_from_f32(d32);
            float dF = kqo_f32_from_f16(d16);
            blk[0] = (uint8_t)(d16 & 0xFF);
            blk[1] = (uint8_t)(d16 >> 8);
            for (int j = 0; j < 32; ++j) {
                int q;
                if (dF == 0.0f) {
                    q = 0;
                } else {
                    q = round_half_away(w[j] / dF);
                    if (q < -127) q = -127;          /* never taken for finite w */
                    if (q > 127) q = 127;
                }
                blk[2 + j] = (uint8_t)(int8_t)q;
            }
        }
    }
    return 0;
}

/* ======================================================================== */
/* Layout change AoS -> planar (byte moves; PQ2_0 code bits placed anew).    */
/* ======================================================================== */

static int fmt_group(int fmt) { return fmt == 1 ? 128 : (fmt == 2 ? 32 : 0); }

int64_t kqo_planar_bytes(int fmt, int64_t N, int64_t K)
{
    int g = fmt_group(fmt);
    if (!g || N < 0 || K <= 0 || K % g) return -1;
    int64_t nb = K / g;
    int64_t tiles = (N + 15) / 16;                      /* 16-row tiles */
    int64_t qs_bytes = tiles * 16 * nb * 32;
    int64_t d_off = (qs_bytes + 255) / 256 * 256;
    int64_t chunks = (nb + 7) / 8;                      /* 8 scales per chunk row */
    return d_off + tiles * chunks * 256;
}

/* The 32 code bytes of block b of row n go to tile (n / 16, b): 16 rows x
 * 32 bytes, row n % 16 at byte 32 * (n % 16), tile (t, b) at byte
 * 512 * (t * nb + b).  Rows past N in the last tile stay zero.  Q8_0 code
 * bytes are copied as they are.  PQ2_0 code word i of a block (its bytes
 * 4i..4i+3, little-endian) holds the same 16 codes as the block's word i
 * [BT 3.1 word view], with code j's low bit at bit 2j as there and its high
 * bit at bit (2j + 3) mod 32 instead of 2j + 1 (pq2_place_codes).  The fp16
 * scales follow at the first 256-byte boundary, in chunks of 16 rows x 8
 * blocks: the scale of block b of row n sits in chunk (n / 16, b / 8), which
 * starts at 256 * ((n / 16) * ceil(nb / 8) + b / 8), at byte
 * 16 * (n % 16) + 2 * (b % 8) of it.  Slots past N or nb stay zero. */
/* One PQ2_0 code word of the planar layout from the block's word view:
 * code j (bits 2j, 2j+1 of `word`) -> low bit at 2j, high bit at (2j+3) % 32. */
static uint32_t pq2_place_codes(uint32_t word)
{
    uint32_t out = 0;
    for (int j = 0; j < 16; ++j) {
        uint32_t q = (word >> (2 * j)) & 3u;
        out |= (q & 1u) << (2 * j);
        out |= (q >> 1) << ((2 * j + 3) % 32);
    }
    return out;
}

int kqo_aos_to_planar(int fmt, const uint8_t *aos, int64_t N, int64_t K,
                      uint8_t *planar)
{
    int g = fmt_group(fmt);
    if (!g || N < 0 || K <= 0 || K % g) return -1;
    int64_t nb = K / g;
    int64_t qs_bytes = (N + 15) / 16 * 16 * nb * 32;
    int64_t d_off = (qs_bytes + 255) / 256 * 256;
    int64_t chunks = (nb + 7) / 8;
    int64_t total = kqo_planar_bytes(fmt, N, K);
    memset(planar, 0, (size_t)total);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = aos + (n * nb + b) * 34;
            uint8_t *dst = planar + ((n / 16) * nb + b) * 512 + (n % 16) * 32;
            memcpy(dst, blk + 2, 32);
            if (fmt == 1) {
                for (int i = 0; i < 8; ++i) {
                    const uint8_t *p = blk + 2 + 4 * i;
                    uint32_t w = (uint32_t)p[0] | ((uint32_t)p[1] << 8) |
                                 ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
                    uint32_t v = pq2_place_codes(w);
                    for (int k = 0; k < 4; ++k) dst[4 * i + k] = (uint8_t)(v >> (8 * k));
                }
            }
            int64_t at = d_off + ((n / 16) * chunks + b / 8) * 256 + (n % 16) * 16 + (b % 8) * 2;
            planar[at + 0] = blk[0];
            planar[at + 1] = blk[1];
        }
    }
    return 0;
}

/* ======================================================================== */
/* Decoders.                                                                */
/* ======================================================================== */

static double blk_scale(const uint8_t *blk)
{
    return (double)kqo_f32_from_f16((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* Byte view [BT 3.1]: element j in byte j/4 at bit offset 2*(j%4); q -> (q-1)*d. */
int kqo_unpack_pq2_aos(const uint8_t *aos, int64_t N, int64_t K, double *W)
{
    if (N < 0 || K <= 0 || K % 128) return -1;
    int64_t nb = K / 128;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = aos + (n * nb + b) * 34;
            double d = blk_scale(blk);
            for (int j = 0; j < 128; ++j) {
                int q = (blk[2 + j / 4] >> (2 * (j % 4))) & 3;
                W[n * K + b * 128 + j] = (double)(q - 1) * d;
            }
        }
    return 0;
}

/* Word view [BT 3.1]: bytes qs[4i..4i+3] as a little-endian u32 hold element
 * 16*i + j at bits 2*j. */
int kqo_unpack_pq2_aos_words(const uint8_t *aos, int64_t N, int64_t K, double *W)
{
    if (N < 0 || K <= 0 || K % 128) return -1;
    int64_t nb = K / 128;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = aos + (n * nb + b) * 34;
            double d = blk_scale(blk);
            for (int i = 0; i < 8; ++i) {
                const uint8_t *p = blk + 2 + 4 * i;
                uint32_t word = (uint32_t)p[0] | ((uint32_t)p[1] << 8) |
                                ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
                for (int j = 0; j < 16; ++j) {
                    int q = (int)((word >> (2 * j)) & 3u);
                    W[n * K + b * 128 + 16 * i + j] = (double)(q - 1) * d;
                }
            }
        }
    return 0;
}

/* Q8_0: w = d * q ([KB]). */
int kqo_unpack_q8_aos(const uint8_t *aos, int64_t N, int64_t K, double *W)
{
    if (N < 0 || K <= 0 || K % 32) return -1;
    int64_t nb = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = aos + (n * nb + b) * 34;
            double d = blk_scale(blk);
            for (int j = 0; j < 32; ++j)
                W[n * K + b * 32 + j] = d * (double)(int8_t)blk[2 + j];
        }
    return 0;
}

/* ======================================================================== */
/* PTQ1_0 [BT 3.2]: the 128 trits of a block (the same values 0, 1, 2 as the  */
/* PQ2_0 codes, same scale) in 24 + 2 bytes of base-3 digits, then the fp16  */
/* scale: 28 bytes.                                                          */
/* ======================================================================== */

/* Where element e of a block lives: trit byte (0..25) and trit position n.
 *   elements   0..79:  byte e % 16 of qs[0..15],  n = e / 16  (5 trits a byte)
 *   elements  80..119: byte 16 + (e - 80) % 8,    n = (e - 80) / 8
 *   elements 120..127: qh byte (e - 120) % 2,      n = (e - 120) / 2 (4 trits) */
static void ptq1_place(int e, int *byte, int *n)
{
    if (e < 80) { *byte = e % 16; *n = e / 16; }
    else if (e < 120) { *byte = 16 + (e - 80) % 8; *n = (e - 80) / 8; }
    else { *byte = 24 + (e - 120) % 2; *n = (e - 120) / 2; }
}

/* A byte holding trits t0..t4 (t0 most significant):
 *   q = ceil(256 * (81 t0 + 27 t1 + 9 t2 + 3 t3 + t4) / 243).
 * A qh byte holds four trits; it is read as five with t4 = 0. */
static uint8_t ptq1_byte(const int t[5])
{
    int v = 81 * t[0] + 27 * t[1] + 9 * t[2] + 3 * t[3] + t[4];
    return (uint8_t)((256 * v + 242) / 243);
}

/* Trit n of byte q: ((q * 3^n) mod 256) * 3 / 256, rounded down. */
static int ptq1_trit(uint8_t q, int n)
{
    int p = 1;
    for (int i = 0; i < n; ++i) p *= 3;
    return (((int)q * p) & 0xFF) * 3 >> 8;
}

int kqo_pq2_to_ptq1_aos(const uint8_t *pq2, int64_t N, int64_t K, uint8_t *ptq1)
{
    if (N < 0 || K <= 0 || K % 128) return -1;
    int64_t nblk = N * (K / 128);
    for (int64_t b = 0; b < nblk; ++b) {
        const uint8_t *in = pq2 + b * 34;
        uint8_t *out = ptq1 + b * 28;
        int t[26][5];
        memset(t, 0, sizeof t);
        for (int e = 0; e < 128; ++e) {
            int c = (in[2 + e / 4] >> (2 * (e % 4))) & 3;   /* [BT 3.1] */
            if (c == 3) return -1;                           /* not a trit */
            int byte, n;
            ptq1_place(e, &byte, &n);
            t[byte][n] = c;
        }
        for (int i = 0; i < 26; ++i) out[i] = ptq1_byte(t[i]);
        out[26] = in[0];                                     /* d, LAST here */
        out[27] = in[1];
    }
    return 0;
}

int kqo_ptq1_to_pq2_aos(const uint8_t *ptq1, int64_t N, int64_t K, uint8_t *pq2)
{
    if (N < 0 || K <= 0 || K % 128) return -1;
    int64_t nblk = N * (K / 128);
    for (int64_t b = 0; b < nblk; ++b) {
        const uint8_t *in = ptq1 + b * 28;
        uint8_t *out = pq2 + b * 34;
        memset(out, 0, 34);
        out[0] = in[26];
        out[1] = in[27];
        for (int e = 0; e < 128; ++e) {
            int byte, n;
            ptq1_place(e, &byte, &n);
            int c = ptq1_trit(in[byte], n);
            out[2 + e / 4] |= (uint8_t)(c << (2 * (e % 4)));
        }
    }
    return 0;
}

int kqo_unpack_ptq1_aos(const uint8_t *ptq1, int64_t N, int64_t K, double *W)
{
    if (N < 0 || K <= 0 || K % 128) return -1;
    int64_t nb = K / 128;
    for (int64_t r = 0; r < N; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = ptq1 + (r * nb + b) * 28;
            double d = (double)kqo_f32_from_f16((uint16_t)(blk[26] | (blk[27] << 8)));
            for (int e = 0; e < 128; ++e) {
                int byte, n;
                ptq1_place(e, &byte, &n);
                W[r * K + b * 128 + e] = (double)(ptq1_trit(blk[byte], n) - 1) * d;
            }
        }
    return 0;
}

/* ======================================================================== */
/* Rotation.                                                                */
/* ======================================================================== */

static int popcount32(uint32_t v)
{
    int c = 0;
    while (v) { c += (int)(v & 1u); v >>= 1; }
    return c;
}

static int valid_block_len(int32_t n)
{
    return n == 0 || (n >= 1 && n <= 1024 && (n & (n - 1)) == 0);
}

/* [BT 4.1]: H[row][col] = (-1)^popcount(row & col), natural (Sylvester) order. */
int kqo_hadamard_matrix(int32_t n, int8_t *H)
{
    if (n < 1 || !valid_block_len(n)) return -1;
    for (int32_t r = 0; r < n; ++r)
        for (int32_t c = 0; c < n; ++c)
            H[(int64_t)r * n + c] = (popcount32((uint32_t)(r & c)) & 1) ? -1 : 1;
    return 0;
}

/* [BT 4.1, 4.2]: R = (1/sqrt(n)) H_n S, applied block-diagonally along K:
 * x' = x (.) s (sign first), then each n-block is multiplied by H_n / sqrt(n). */
int kqo_rotate(const double *x, int64_t M, int64_t K, int32_t n,
               const int8_t *signs, double *xr)
{
    if (!valid_block_len(n) || M < 0 || K <= 0) return -1;
    if (n > 0 && K % n) return -1;
    double *sx = (double *)malloc(sizeof(double) * (size_t)K);
    if (!sx) return -1;
    int8_t *H = NULL;
    if (n > 0) {
        H = (int8_t *)malloc((size_t)n * (size_t)n);
        if (!H) { free(sx); return -1; }
        kqo_hadamard_matrix(n, H);
    }
    double scale = n > 0 ? 1.0 / sqrt((double)n) : 1.0;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            sx[k] = (signs && signs[k] < 0) ? -x[m * K + k] : x[m * K + k];
        if (n == 0) {
            memcpy(xr + m * K, sx, sizeof(double) * (size_t)K);
            continue;
        }
        for (int64_t b = 0; b < K / n; ++b) {
            const double *xb = sx + b * n;
            for (int32_t r = 0; r < n; ++r) {
                double acc = 0.0;
                for (int32_t c = 0; c < n; ++c)
                    acc += (double)H[(int64_t)r * n + c] * xb[c];
                xr[m * K + b * n + r] = scale * acc;
            }
        }
    }
    free(H);
    free(sx);
    return 0;
}

/* ======================================================================== */
/* Product.                                                                 */
/* ======================================================================== */

void kqo_matmul(const double *W, const double *xr, int64_t M, int64_t N,
                int64_t K, double *y, double *bnd)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = W[n * K + k] * xr[m * K + k];
                acc += p;
                abs_acc += fabs(p);
            }
            y[m * N + n] = acc;
            if (bnd) bnd[m * N + n] = abs_acc;
        }
    }
}

int kqo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void kqo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int kqo_gemv_aos(int fmt, const uint8_t *aos, int64_t N, int64_t K,
                 const float *x, int64_t M, int32_t block_len,
                 const int8_t *signs, double *y, double *bnd)
{
    int g = fmt_group(fmt);
    if (!g || N < 0 || M < 1 || K <= 0 || K % g) return -1;
    if (!valid_block_len(block_len) || (block_len > 0 && K % block_len)) return -1;
    double *Wd = (double *)malloc(sizeof(double) * (size_t)(N * K));
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K));
    double *xr = (double *)malloc(sizeof(double) * (size_t)(M * K));
    int rc = -1;
    if (Wd && xd && xr) {
        rc = (fmt == 1) ? kqo_unpack_pq2_aos(aos, N, K, Wd)
                        : kqo_unpack_q8_aos(aos, N, K, Wd);
        for (int64_t i = 0; i < M * K; ++i) xd[i] = (double)x[i];
        if (rc == 0) rc = kqo_rotate(xd, M, K, block_len, signs, xr);
        if (rc == 0) kqo_matmul(Wd, xr, M, N, K, y, bnd);
    }
    free(Wd); free(xd); free(xr);
    return rc;
}
