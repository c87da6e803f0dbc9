// gemv.hip -- quantized GEMV (M = 1..8 activation rows) on the CDNA4 matrix cores.
//
// y[m][n] = sum_k deq(W)[n][k] * x'[m][k],   x' = blockwise rotation of x
//   PQ2_0 deq = (q-1)*d per 128-group (Bonsai ternary g128 page, sec. 3.1);
//   Q8_0  deq = d*q per 32-group (Kipp pages, "Weight quantization");
//   x' = (1/sqrt(n)) H_n (s (.) x) per n-block (Bonsai page, sec. 4.1-4.2).
//
// gfx950 design
// -------------
// The product is bandwidth-bound, so the arithmetic has to stay well under
// one vector instruction per weight.  The multiply-adds go to the matrix
// cores and the vector ALUs only unpack:
// * PQ2_0.  Three bit operations per stored 32-bit word turn 16 2-bit codes
//   into 16 signed E2M1 (fp4) operands of value (c - 1) / 2, so that
//   v_mfma_scale_f32_16x16x128_f8f6f4 multiplies 16 weight rows x 128 codes
//   (one quantization group) by a 16-row operand that holds x' as four e5m2
//   terms (|x' - (t0 + t1 + t2 + t3)| <= 2^-12 |x'|) for up to four
//   activation rows.  Each group of x' is scaled by its own power of two
//   first, so its range suits e5m2.  A zero weight is a zero operand: the
//   matrix core aligns the products of one instruction to the largest of
//   them, so only weights that count may set that scale.
// * Q8_0, up to four activation rows.  The int8 weights go into
//   v_mfma_i32_16x16x32_i8 as loaded; x' enters as four int8 digits of 7 bits
//   under a power-of-two scale per row, the integer sums convert to fp32
//   exactly, and one fma_mix per value applies the fp16 scale.  Five to eight
//   rows: each int8 converts to bf16 exactly and x' is split into bf16 hi + lo
//   parts (2^-17 relative), so that one v_mfma_f32_16x16x32_bf16 covers 16
//   weight rows x one 32-group for all rows.
// * Work split.  A workgroup owns a K-slice and a range of 16-row blocks.  Its
//   waves split the K-slice (GS groups each) and hold their part of the
//   activation operand in registers for the whole kernel.  Every wave
//   streams the same row blocks: one 16-byte buffer load per lane covers 16
//   rows x 64 bytes (a pair of groups), and one permlane32 swap per register
//   puts the pair into MFMA operand order (lane block kb ends up with bytes
//   {0, 16, 8, 24}[kb] + 0..7 of each group; the activation operand uses the
//   same K order).  Weight loads run D row blocks ahead of the arithmetic;
//   the first ones are issued right after the activation loads, so the
//   prologue overlaps the first weight fetches.  Buffer-resource range
//   checks return zeros past the last row, so the loads need no branches.
// * Prologue.  PQ2_0: every wave rotates and splits its own 1024-element
//   K-range, butterflies in registers and across lanes (DPP, permlane
//   swaps), without workgroup barriers.  Q8_0: the workgroup stages its
//   K-slice of x in LDS (with LDS butterflies for wide rotation blocks) and
//   each lane converts its operand from there.
// * Reduction.  After the MFMAs each lane's accumulators belong to one
//   (weight row, activation row); the wave partials go through LDS and are
//   added in wave order every RBR row blocks (deterministic, no atomics).
// * Split-K.  blockIdx.y selects one of S contiguous K-slices made of whole
//   rotation blocks; each writes fp32 partials [S][M][N] that a second kernel
//   adds in ascending s.
#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRB = 16;  // weight rows per block (MFMA width)
// Weight loads go through one buffer resource per plane and workgroup, based
// at its first row and at most kMaxWgBytes long.  Row blocks past the
// workgroup's range are loaded at kFarRows, outside that range, so they
// return zeros without touching memory; every offset stays below 2^31 + 2^30,
// clear of wrap-around in the range check.
constexpr uint32_t kFarRows = 0x40000000u;
constexpr int64_t kMaxWgBytes = int64_t(1) << 29;
constexpr int kLdsBudget = 160 * 1024;
constexpr int kTargetWGs = 256;  // one workgroup per CU
constexpr int kEarlyWave = 8;

// One weight set of a multi-set call: its planes, output and row blocks, and
// the first workgroup of the grid that works on it.
struct GemvSet {
  const uint8_t* qs;
  const uint8_t* dpl;
  float* out;
  int64_t N;
  int q_base, q_rem;  // row units per workgroup of this set (see row_unit)
  int wg0;
  int pad;
};

struct GemvArgs {
  const uint8_t* qs;
  const uint8_t* dpl;
  const float* x;        // activations [M][K]
  const int8_t* signs;   // K entries, or null
  float* out;            // y [M][N] (S == 1) or partials [S][M][N]
  int64_t N, K;
  uint32_t row_bytes;    // qs bytes per weight row (32 per group)
  uint32_t d_tile_bytes; // scale bytes per 16-row tile (256 per 8 groups)
  int G;                 // groups per row
  int U;                 // groups per rotation block (slices hold whole blocks)
  int S;                 // K slices
  int total_rb;          // 16-row blocks
  int grid_x;
  int q_base, q_rem;     // workgroup b owns row units [b*q_base + min(b, q_rem), next)
  int row_unit;          // rows per unit: 4 or 16
  int u_base, u_rem;     // slice s owns rotation blocks [s*u_base + min(s, u_rem), next)
  int log2n;             // rotation block length (0: no transform)
  float inv_sqrt_n;
  int nsets;             // 1, or up to kMaxSets weight sets sharing x (then S == 1)
  GemvSet set[kMaxSets];
};

// The rows of this workgroup: its weight set (a uniform choice), that set's
// planes and output, and its range of 16-row blocks.  Every set sees the same
// activation slices and launch shape, so its outputs are bit-identical to a
// call for that set alone.  (The arguments are never written: a modified
// copy of them went through scratch memory.)
struct WgRows {
  const uint8_t* qs;
  const uint8_t* dpl;
  float* out;
  int64_t N;
  int r0, r1;    // its rows [r0, r1)
  int rb0, rb1;  // the 16-row blocks that hold them
};
// Rows are handed out in units of row_unit rows.  Q8_0 uses 4 (one 128-byte
// line of a 16-row code tile), so that every workgroup streams the same
// bytes: with whole 16-row blocks, 1088 blocks over 256 workgroups left a
// quarter of them a fifth block in place of 4.25, and those set the
// kernel's time (18.5 -> 18.0 us at M = 1, 27.0 -> 26.1 us at M = 8).  A
// workgroup's first and last blocks may then hold rows of its neighbours:
// its lanes of those rows load nothing and write nothing.  PQ2_0 uses whole
// blocks (16): its partial blocks cost a full block of decode and matrix
// work for half the bytes, which measured slower (5.43 against 5.34 us at
// 10240 rows).
__host__ __device__ __forceinline__ int part_start(int i, int base, int rem);
// MULTI: a kernel instance for several sets (one-set calls read no set
// fields, so their prologue starts as early as before).
template <bool MULTI>
__device__ __forceinline__ WgRows wg_rows(const GemvArgs& a) {
  const int b = (int)blockIdx.x;
  WgRows w;
  if constexpr (!MULTI) {
    w.qs = a.qs;
    w.dpl = a.dpl;
    w.out = a.out;
    w.N = a.N;
    w.r0 = a.row_unit * part_start(b, a.q_base, a.q_rem);
    const int64_t e = (int64_t)a.row_unit * part_start(b + 1, a.q_base, a.q_rem);
    w.r1 = (int)(e < a.N ? e : a.N);
    w.rb0 = w.r0 / kRB;
    w.rb1 = (w.r1 + kRB - 1) / kRB;
    return w;
  }
  const int s = (1 < a.nsets && b >= a.set[1].wg0) + (2 < a.nsets && b >= a.set[2].wg0) +
                (3 < a.nsets && b >= a.set[3].wg0);
  static_assert(kMaxSets == 4, "the selection below lists the sets");
#define KQ_PICK(f) (s == 0 ? a.set[0].f : s == 1 ? a.set[1].f : s == 2 ? a.set[2].f : a.set[3].f)
  w.qs = KQ_PICK(qs);
  w.dpl = KQ_PICK(dpl);
  w.out = KQ_PICK(out);
  w.N = KQ_PICK(N);
  const int base = KQ_PICK(q_base), rem = KQ_PICK(q_rem), bx = b - KQ_PICK(wg0);
#undef KQ_PICK
  w.r0 = a.row_unit * part_start(bx, base, rem);
  const int64_t e = (int64_t)a.row_unit * part_start(bx + 1, base, rem);
  w.r1 = (int)(e < w.N ? e : w.N);
  w.rb0 = w.r0 / kRB;
  w.rb1 = (w.r1 + kRB - 1) / kRB;
  return w;
}

// The arguments a wave needs before its first loads, passed as the kernel's
// leading scalar parameters: the first 14 dwords of a kernel's arguments are
// preloaded into scalar registers before its waves start, so the activation
// and weight loads go out without waiting for a scalar load of the argument
// block.  The rest stays in GemvArgs (loaded behind the first vector loads).
struct GemvHead {
  const uint8_t* qs;
  const uint8_t* dpl;
  const float* x;
  const int8_t* signs;
  int q_base, q_rem;  // 16-row blocks per workgroup (one weight set)
  int n;              // rows (fits 32 bits)
  int G;              // groups per row: 32 G code bytes a row, 256 ceil(G/8) scale bytes a tile
  int u_br;           // K slices of whole rotation blocks: u_base | u_rem << 16
  int unw;            // groups per rotation block | waves per workgroup << 8
};
#define KQ_HEAD_PARAMS                                                                        \
  const uint8_t *__restrict__ h_qs, const uint8_t *__restrict__ h_dpl,                       \
      const float *__restrict__ h_x, const int8_t *__restrict__ h_sg, int h_qb, int h_qr,    \
      int h_n, int h_g, int h_ubr, int h_unw
#define KQ_HEAD_MAKE {h_qs, h_dpl, h_x, h_sg, h_qb, h_qr, h_n, h_g, h_ubr, h_unw}
#define KQ_HEAD_ARGS(h)                                                                       \
  (h).qs, (h).dpl, (h).x, (h).signs, (h).q_base, (h).q_rem, (h).n, (h).G, (h).u_br, (h).unw
static_assert(sizeof(GemvHead) == 56, "the head is 14 preloaded dwords");

__device__ __forceinline__ WgRows wg_rows_head(const GemvHead& h) {
  const int b = (int)blockIdx.x;
  WgRows w;
  w.qs = h.qs;
  w.dpl = h.dpl;
  w.out = nullptr;
  w.N = h.n;
  w.r0 = kRB * part_start(b, h.q_base, h.q_rem);
  const int e = kRB * part_start(b + 1, h.q_base, h.q_rem);
  w.r1 = e < h.n ? e : h.n;
  w.rb0 = w.r0 / kRB;
  w.rb1 = (w.r1 + kRB - 1) / kRB;
  return w;
}

// ---------------------------------------------------------------------------
// shared device helpers

// The activation's address and the workgroup's weight planes as scalar
// operands of an empty asm right after the row range is known: without it
// the compiler loads them from the kernel arguments only where first used,
// each behind its own wait, and the first weight loads went out about 0.4 us
// after a wave started.
__device__ __forceinline__ void args_in_one_batch(const GemvArgs& a, const WgRows& w) {
  asm volatile("" ::"s"(a.x), "s"(w.qs), "s"(w.dpl));
}

__device__ __forceinline__ uint2 buffer_load_8B(BufRsrc r, uint32_t off) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v.x, v.y);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// value of lane (lane ^ DIST), DIST in {1, 2, 4, 8, 16, 32}
template <int DIST>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (DIST == 1) {
    return dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (DIST == 2) {
    return dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (DIST == 4) {
    return dpp<0x1B>(dpp<0x141>(v));  // half-row mirror (i^7), then quad_perm i^3
  } else if constexpr (DIST == 8) {
    return dpp<0x141>(dpp<0x140>(v));  // row mirror (i^15), then half-row mirror (i^7)
  } else if constexpr (DIST == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                    false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 16) ? p[0] : p[1]);
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                    false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? p[0] : p[1]);
  }
}

// butterfly across lanes at distance DIST: the lower lane keeps a + b, the
// upper one a - b (natural-order Sylvester stage)
template <int DIST, int NV>
__device__ __forceinline__ void lane_butterfly(float (&v)[NV]) {
  const float sgn = (threadIdx.x & DIST) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = fmaf(sgn, v[i], xor_lane<DIST>(v[i]));
}

// The butterfly at distance 1 or 2 (inside a quad) in one instruction per
// value: v_fmac_f32_dpp adds the partner's value times s, +1 on the lower
// lane and -1 on the upper one, so the lower lane gets a + b and the upper
// one b - a, the negative of the Sylvester stage's a - b.  Stages commute with
// a sign that depends only on lane bits they do not pair, so the whole
// transform comes out as D (H x) with D = -1 on lanes of odd parity in the
// bits of these stages; the caller folds D into its per-element scale
// (quad_stage_sign).  Two instructions per value (DPP move, FMA) before.
// One asm block with its own hazard wait (a DPP read of a register written
// by the vector ALU needs two wait states).
template <int DIST, int NV>
__device__ __forceinline__ void quad_butterfly(float (&v)[NV]) {
  static_assert(DIST == 1 || DIST == 2, "quad distances");
  static_assert(NV == 8 || NV == 16, "one block of 8 or 16 values");
  const float s = (threadIdx.x & DIST) ? -1.f : 1.f;
#define KQ_QB(P)                                                                          \
  asm volatile("s_nop 1\n\t"                                                             \
               "v_fmac_f32_dpp %0, %0, %8 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %1, %1, %8 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %2, %2, %8 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %3, %3, %8 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %4, %4, %8 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %5, %5, %8 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %6, %6, %8 quad_perm:" P " row_mask:0xf bank_mask:0xf\n\t" \
               "v_fmac_f32_dpp %7, %7, %8 quad_perm:" P " row_mask:0xf bank_mask:0xf"      \
               : "+v"(v[i]), "+v"(v[i + 1]), "+v"(v[i + 2]), "+v"(v[i + 3]), "+v"(v[i + 4]), \
                 "+v"(v[i + 5]), "+v"(v[i + 6]), "+v"(v[i + 7])                             \
               : "v"(s))
#pragma unroll
  for (int i = 0; i < NV; i += 8) {
    if constexpr (DIST == 1) KQ_QB("[1,0,3,2]");
    else KQ_QB("[2,3,0,1]");
  }
#undef KQ_QB
}
// D of quad_butterfly for a rotation of 2^log2n elements, EPL = 2^LOG_EPL per lane
template <int LOG_EPL>
__device__ __forceinline__ float quad_stage_sign(int log2n) {
  const int lane = threadIdx.x;
  const int bits = (log2n > LOG_EPL ? 1 : 0) | (log2n > LOG_EPL + 1 ? 2 : 0);
  return (__builtin_popcount(lane & bits) & 1) ? -1.f : 1.f;
}

// The same butterfly at distance 4 or 8, where the lower and the upper lanes
// of each pair fall in different DPP banks (groups of 4 lanes of a row): a
// bank-masked add writes the lower lanes (partner + own) and a bank-masked
// subtract the upper ones (partner - own), two instructions per value.  The
// compiler inserts no hazard wait states around inline assembly, so each block
// brings its own: a DPP read of a register written by the vector ALU needs two.
template <int DIST, int NV>
__device__ __forceinline__ void bank_butterfly(float (&v)[NV]) {
  static_assert(DIST == 4 || DIST == 8, "bank-masked butterflies pair lanes 4 or 8 apart");
  static_assert(NV % 4 == 0, "blocks of four values");
#pragma unroll
  for (int i = 0; i < NV; i += 4) {
    float r0, r1, r2, r3;
    if constexpr (DIST == 4) {
      asm volatile(
          "s_nop 1\n\t"
          "v_add_f32_dpp %0, %4, %4 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
          "v_add_f32_dpp %1, %5, %5 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
          "v_add_f32_dpp %2, %6, %6 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
          "v_add_f32_dpp %3, %7, %7 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
          "v_sub_f32_dpp %0, %4, %4 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
          "v_sub_f32_dpp %1, %5, %5 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
          "v_sub_f32_dpp %2, %6, %6 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
          "v_sub_f32_dpp %3, %7, %7 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
          "s_nop 1"
          : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
          : "v"(v[i]), "v"(v[i + 1]), "v"(v[i + 2]), "v"(v[i + 3]));
    } else {
      asm volatile(
          "s_nop 1\n\t"
          "v_add_f32_dpp %0, %4, %4 row_shl:8 row_mask:0xf bank_mask:0x3\n\t"
          "v_add_f32_dpp %1, %5, %5 row_shl:8 row_mask:0xf bank_mask:0x3\n\t"
          "v_add_f32_dpp %2, %6, %6 row_shl:8 row_mask:0xf bank_mask:0x3\n\t"
          "v_add_f32_dpp %3, %7, %7 row_shl:8 row_mask:0xf bank_mask:0x3\n\t"
          "v_sub_f32_dpp %0, %4, %4 row_shr:8 row_mask:0xf bank_mask:0xc\n\t"
          "v_sub_f32_dpp %1, %5, %5 row_shr:8 row_mask:0xf bank_mask:0xc\n\t"
          "v_sub_f32_dpp %2, %6, %6 row_shr:8 row_mask:0xf bank_mask:0xc\n\t"
          "v_sub_f32_dpp %3, %7, %7 row_shr:8 row_mask:0xf bank_mask:0xc\n\t"
          "s_nop 1"
          : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
          : "v"(v[i]), "v"(v[i + 1]), "v"(v[i + 2]), "v"(v[i + 3]));
    }
    v[i] = r0; v[i + 1] = r1; v[i + 2] = r2; v[i + 3] = r3;
  }
}

// power-of-two exponent e that puts bound * 2^e in [2^14, 2^15), read from
// the binary32 exponent field (a subnormal bound takes the maximum e; zero,
// infinity and NaN give 0)
__device__ __forceinline__ int range_exponent(float bound) {
  const uint32_t ef = (__float_as_uint(bound) >> 23) & 0xFFu;
  if (!(bound > 0.f) || ef == 0xFFu) return 0;
  const int e = 14 - ((int)ef - 127);
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}

// bf16 bits (in the upper half of a binary32) of an int8 byte: exact
__device__ __forceinline__ uint32_t i8_as_f32bits(uint32_t w, int byte) {
  return __float_as_uint((float)(int8_t)(w >> (8 * byte)));
}
// [lo.upper16, hi.upper16] -- two bf16 values from two binary32 bit patterns
__device__ __forceinline__ uint32_t bf16_pair(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Swap the two groups of a loaded pair into MFMA operand order (see above).
// Written as inline assembly (the swap rewrites both registers in place, and
// the builtin's register constraints made the compiler copy loaded registers
// at the loop head, waiting for loads still in flight).  The compiler does
// not insert hazard wait states around inline assembly, so the block carries
// its own: a vector ALU write of a register followed by a permlane read of it
// needs them.
__device__ __forceinline__ void pair_to_operands(const uint4& v, uint2& g0, uint2& g1) {
  uint32_t x = v.x, y = v.y, z = v.z, w = v.w;
  asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\ts_nop 4"
               : "+v"(x), "+v"(z), "+v"(y), "+v"(w));
  g0 = make_uint2(x, y);
  g1 = make_uint2(z, w);
}

// The 16 2-bit codes of one stored word (code j: b0 at bit 2j, b1 at bit
// (2j + 3) mod 32, see pq2_store_word) as signed E2M1 (fp4) operands of value
// (c - 1) / 2: code 0 -> -0.5 (1001), 1 -> -0 (1000), 2 -> +0.5 (0001).  Code
// 3 is not a PQ2_0 value (the format maps only codes 0, 1 and 2, and its
// packer never writes 3); it becomes +0 (0000).  Even codes go to the nibbles
// of `ev`, odd ones to those of `od` (code 2i and 2i+1 to nibble i).  Nibble
// bits: [3] = ~b1, [2] = [1] = 0, [0] = ~b0.
// Signed operands keep every product of a zero weight at zero: the matrix
// core sums the products of one instruction aligned to the largest of them,
// so the smaller ones keep only about 2^-17 of it, and that must be measured
// against the output's own sum of |w x'| (a form with a constant offset added
// to every weight lets a large activation element with a zero weight set that
// scale).
// truth table of v_bitop3_b32 for f(a, b, c): bit (a << 2 | b << 1 | c)
template <typename F>
constexpr uint32_t bitop3_table(F f) {
  uint32_t t = 0;
  for (int i = 0; i < 8; ++i) t |= (f((i >> 2) & 1, (i >> 1) & 1, i & 1) & 1u) << i;
  return t;
}
__device__ __forceinline__ void ternary_fp4(uint32_t w, uint32_t& ev, uint32_t& od) {
  // The even codes' bits already sit at nibble bits 0 and 3, the odd codes'
  // two places up: one v_bitop3_b32 (~x & m) per half, after a rotate
  // (v_alignbit_b32) for the odd half.  Three instructions for 16 codes.
  constexpr uint32_t M03 = 0x99999999u;
  constexpr uint32_t kSel = bitop3_table([](int m, int x, int) { return m && !x; });
  ev = __builtin_amdgcn_bitop3_b32(M03, w, w, kSel);
  const uint32_t r = __builtin_amdgcn_alignbit(w, w, 2);  // w rotated down by two
  od = __builtin_amdgcn_bitop3_b32(M03, r, r, kSel);
}

// start of part i when parts of `base` items get one more for i < rem
__host__ __device__ __forceinline__ int part_start(int i, int base, int rem) {
  return i * base + (i < rem ? i : rem);
}
// K slice s of S (whole rotation blocks of U groups)
__device__ __forceinline__ void slice_groups(const GemvArgs& a, int s, int& g0, int& g1) {
  g0 = part_start(s, a.u_base, a.u_rem) * a.U;
  g1 = part_start(s + 1, a.u_base, a.u_rem) * a.U;
}

// fixed-order sum of the wave partials of one round into y (or split partials);
// each wave leaves KS partials per output, [NW][RBR][M][KS][16]
__device__ __forceinline__ void reduce_round(const WgRows& a, const float* part, int NW, int RBR,
                                             int M, int KS, int rb0, int nrb, int round, int s) {
  const float* pr = part + (round & 1) * NW * RBR * M * KS * kRB;
  for (int it = threadIdx.x; it < RBR * M * kRB; it += blockDim.x) {
    const int jr = it / (M * kRB), m = (it / kRB) % M, r = it % kRB;
    const int j = round * RBR + jr;
    const int row = (rb0 + j) * kRB + r;
    if (j < nrb && row >= a.r0 && row < a.r1) {
      float t = 0.f;
      for (int w = 0; w < NW; ++w)
        for (int k = 0; k < KS; ++k) t += pr[(((w * RBR + jr) * M + m) * KS + k) * kRB + r];
      a.out[((int64_t)s * M + m) * a.N + row] = t;
    }
  }
}

// One activation row: each wave leaves one partial per output row (its four
// lane blocks already added), [RBR][16 rows][NWP wave slots]; the slots of
// waves past NW hold zeros (written in the prologue), and the NWP slots are
// added as a fixed tree, read as NWP / 4 16-byte words.
template <int NWP>
__device__ __forceinline__ float sum_slots(const float* pr) {
  const float4* p = reinterpret_cast<const float4*>(pr);
  float v[NWP];
#pragma unroll
  for (int q = 0; q < NWP / 4; ++q) {
    const float4 f = p[q];
    v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
  }
#pragma unroll
  for (int h = 1; h < NWP; h *= 2)
#pragma unroll
    for (int w = 0; w + h < NWP; w += 2 * h) v[w] += v[w + h];
  return v[0];
}
template <int NWP>
__device__ __forceinline__ void reduce_round_one(const WgRows& a, const float* part, int RBR,
                                                 int rb0, int nrb, int round, int s) {
  const float* pr = part + (round & 1) * RBR * kRB * NWP;
  for (int it = threadIdx.x; it < RBR * kRB; it += blockDim.x) {
    const int jr = it / kRB, r = it % kRB;
    const int j = round * RBR + jr;
    const int row = (rb0 + j) * kRB + r;
    if (j < nrb && row >= a.r0 && row < a.r1) a.out[(int64_t)s * a.N + row] = sum_slots<NWP>(pr + it * NWP);
  }
}

// ---------------------------------------------------------------------------
// Weight loads of one row block for one wave (shared by every GEMV kernel and
// by its loads-only twin): the codes of the wave's GS groups, one 16-byte
// streamed load per lane and pair of groups, and the GS fp16 scales of the
// lane's row.  ro / rod: byte offsets of the row block in the code and scale
// resources (kFarRows past the workgroup's range, which returns zeros).

template <int GS>
struct WBuf {
  uint4 q[GS / 2];
  uint32_t d[GS / 2];
};

// qoff: per pair, the lane's code offset inside a row block (or kOutOfRange);
// doff: the lane's offset of its first scale inside a 16-row scale tile;
// gfirst: absolute index of the wave's first group; DALIGN: gfirst % 8 == 0
// for GS >= 8, gfirst % 4 == 0 for GS == 4 (whole aligned runs of scales).
template <int GS, bool DALIGN>
__device__ __forceinline__ void issue_row_block(WBuf<GS>& b, BufRsrc rq, BufRsrc rd,
                                                const uint32_t (&qoff)[GS / 2], uint32_t doff,
                                                int gfirst, int r16, uint32_t ro, uint32_t rod) {
#pragma unroll
  for (int q = 0; q < GS / 2; ++q) b.q[q] = buffer_load_16B_stream(rq, qoff[q] + ro);
  if constexpr (DALIGN) {
    if constexpr (GS == 4) {
      const uint2 t = buffer_load_8B(rd, doff + rod);
      b.d[0] = t.x; b.d[1] = t.y;
    } else {
#pragma unroll
      for (int i = 0; i < GS / 8; ++i) {
        const uint4 t = buffer_load_16B(rd, doff + rod + 256u * i);
        b.d[4 * i] = t.x; b.d[4 * i + 1] = t.y; b.d[4 * i + 2] = t.z; b.d[4 * i + 3] = t.w;
      }
    }
  } else {
    // one scale per load, each at its own chunk and slot
    const uint32_t rbase = (uint32_t)r16 * 16u + rod;
#pragma unroll
    for (int i = 0; i < GS / 2; ++i) {
      const int ge = gfirst + 2 * i, go = ge + 1;
      const uint32_t oe = (uint32_t)(ge >> 3) * 256u + (uint32_t)(ge & 7) * 2u;
      const uint32_t oo = (uint32_t)(go >> 3) * 256u + (uint32_t)(go & 7) * 2u;
      b.d[i] = buffer_load_2B(rd, rbase + oe) | (buffer_load_2B(rd, rbase + oo) << 16);
    }
  }
}

// The same loads in parts, for a buffer that is refilled while it is read:
// the codes of pair q, and the scales of groups 8c .. 8c + 7 (whole aligned
// runs, DALIGN) or of pair c alone (otherwise).
template <int GS>
__device__ __forceinline__ void issue_codes(WBuf<GS>& b, int q, BufRsrc rq, uint32_t qo, uint32_t ro) {
  b.q[q] = buffer_load_16B_stream(rq, qo + ro);
}
template <int GS, bool DALIGN>
__device__ __forceinline__ void issue_scales(WBuf<GS>& b, int c, BufRsrc rd, uint32_t doff, int gfirst,
                                             int r16, uint32_t rod) {
  if constexpr (DALIGN) {
    static_assert(GS >= 8, "scale runs of eight groups");
    const uint4 t = buffer_load_16B(rd, doff + rod + 256u * c);
    b.d[4 * c] = t.x; b.d[4 * c + 1] = t.y; b.d[4 * c + 2] = t.z; b.d[4 * c + 3] = t.w;
  } else {
    const uint32_t rbase = (uint32_t)r16 * 16u + rod;
    const int ge = gfirst + 2 * c, go = ge + 1;
    const uint32_t oe = (uint32_t)(ge >> 3) * 256u + (uint32_t)(ge & 7) * 2u;
    const uint32_t oo = (uint32_t)(go >> 3) * 256u + (uint32_t)(go & 7) * 2u;
    b.d[c] = buffer_load_2B(rd, rbase + oe) | (buffer_load_2B(rd, rbase + oo) << 16);
  }
}

// ---------------------------------------------------------------------------
// PQ2_0

// EPL activation elements per lane in the prologue: 8 (half a packed code
// word per lane, GS = 4 groups per wave) for rotation blocks up to 512, 16 (a
// whole word, GS = 8) for 1024-blocks, which must sit inside one wave.
template <int EPL>
struct Pq2Cfg {
  static constexpr int LOG_EPL = EPL == 8 ? 3 : 4;
  static constexpr int GS = EPL / 2;     // groups per wave: 64 lanes x EPL elements
  static constexpr int LPG = 128 / EPL;  // lanes per 128-group
  static constexpr int LPW = 16 / EPL;   // lanes per packed code word
  static constexpr int D = 3;            // row blocks of weight loads in flight (4: 5.40 us at
                                         // 10240 rows, 56.5 us at 248320; 3: 5.35, 55.5)
  static constexpr int RBR = 8;          // row blocks per reduction round
  static constexpr int MAXW = EPL == 8 ? 12 : 8;  // 12: up to 168 VGPRs per lane
};

// LDS bytes: per wave [GS][M][4 terms][4 kb][32 B] operand bytes, then the
// partials [2][NW][RBR][M][KS][16] floats, then 32 zero bytes (the operand of
// unused rows and groups).  KS = 4 for one activation row (the four lane
// blocks hold one term each), else 1.
__host__ __device__ inline int pq2_ks(int M) { return M == 1 ? 4 : 1; }
__host__ __device__ inline int pq2_lds_part_offset(int M, int NW, int GS) { return NW * GS * M * 512; }
// waves' slots per output row in the one-row partials (a multiple of four)
__host__ __device__ constexpr int pq2_nwp(int GS) { return GS == 4 ? 12 : 8; }
__host__ __device__ inline int pq2_lds_zero_offset(int M, int NW, int GS) {
  return pq2_lds_part_offset(M, NW, GS) +
         (M == 1 ? 2 * 8 * kRB * pq2_nwp(GS) * 4 : 2 * NW * 8 * M * pq2_ks(M) * kRB * 4);
}
__host__ __device__ inline int pq2_lds_bytes(int M, int NW, int GS) { return pq2_lds_zero_offset(M, NW, GS) + 32; }

// Unnormalised Sylvester transform of 2^L consecutive elements held by
// 2^(L - LOG_EPL) lanes, 2^LOG_EPL per lane: the element bits inside a lane
// first, then those across lanes (distance 1..32).  Stages of a transform
// commute, so any order gives H_n.
template <int LOG_EPL, int L, int NV>
__device__ __forceinline__ void rotate_fixed(float (&v)[NV]) {
  constexpr int IN = L < LOG_EPL ? L : LOG_EPL;
#pragma unroll
  for (int st = 0; st < IN; ++st) {
    const int h = 1 << st;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if ((i & h) == 0) {
        const float p0 = v[i], p1 = v[i + h];
        v[i] = p0 + p1;
        v[i + h] = p0 - p1;
      }
  }
  if constexpr (L > LOG_EPL) quad_butterfly<1>(v);
  if constexpr (L > LOG_EPL + 1) quad_butterfly<2>(v);
  if constexpr (L > LOG_EPL + 2) bank_butterfly<4>(v);
  if constexpr (L > LOG_EPL + 3) bank_butterfly<8>(v);
  if constexpr (L > LOG_EPL + 4) lane_butterfly<16>(v);
  if constexpr (L > LOG_EPL + 5) lane_butterfly<32>(v);
}
// run-time block length: one branch, then a straight-line transform
template <int LOG_EPL, int NV>
__device__ __forceinline__ void rotate(float (&v)[NV], int log2n) {
  switch (log2n) {
    case 1: rotate_fixed<LOG_EPL, 1>(v); break;
    case 2: rotate_fixed<LOG_EPL, 2>(v); break;
    case 3: rotate_fixed<LOG_EPL, 3>(v); break;
    case 4: rotate_fixed<LOG_EPL, 4>(v); break;
    case 5: rotate_fixed<LOG_EPL, 5>(v); break;
    case 6: rotate_fixed<LOG_EPL, 6>(v); break;
    case 7: rotate_fixed<LOG_EPL, 7>(v); break;
    case 8: rotate_fixed<LOG_EPL, 8>(v); break;
    case 9: rotate_fixed<LOG_EPL, 9>(v); break;
    case 10: if constexpr (LOG_EPL + 6 >= 10) rotate_fixed<LOG_EPL, 10>(v); break;
    default: break;  // 0: no transform
  }
}
// max (of values >= 0) over the LPG lanes of one 128-group (8 lanes:
// a half row, 16: a row).  Pairs: xor 1, xor 2 within quads, then the half-row
// and row mirrors (lane i with 7 - i, 15 - i), which pair each quad with the
// other quad and each half with the other half; both lanes of a pair combine
// the same two values, so every lane ends with the same bits.  Non-negative
// binary32 values order like their bit patterns, so the max is an integer one.
template <int LPG>
__device__ __forceinline__ float group_max(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));
  if constexpr (LPG == 16) u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, true));
  return __uint_as_float(u);
}

// FEW: every workgroup owns at most D row blocks (the host checks), so all of
// them are in flight once the prologue has run and there is no loop.  A
// separate instance: with the loop in the same function the compiler's
// memory waits before the first row block covered nearly every later load.
template <int M, bool DALIGN, int EPL, bool MULTI, bool FEW>
__global__ __launch_bounds__(Pq2Cfg<EPL>::MAXW * 64) void gemv_pq2_kernel(KQ_HEAD_PARAMS, GemvArgs a) {
  const GemvHead h = KQ_HEAD_MAKE;
  using C = Pq2Cfg<EPL>;
  constexpr int GS = C::GS, D = C::D, RBR = C::RBR, LPG = C::LPG;
  constexpr int TILES = (M + 3) / 4;
  constexpr int MPRE = EPL == 8 ? (M < 4 ? M : 4) : 1;  // activation rows loaded before the weights
  // One activation row: operand row 4*t holds term t, so lane block kb ends
  // with term kb of its weight row in the first accumulator, and the group's
  // power-of-two range scale rides on the MFMA's own A scale (E8M0).  More
  // rows: operand row 4*m + t, every accumulator used, scales applied after.
  constexpr bool ONE = M == 1;
  constexpr int KS = ONE ? 4 : 1;
  constexpr int NWP = pq2_nwp(GS);
  static_assert(NWP >= C::MAXW && NWP % 4 == 0, "a slot for every wave");
  extern __shared__ __align__(16) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // waves per workgroup from the preloaded head (blockDim comes from a
  // scalar load of the dispatch's implicit arguments, and its wait landed
  // before the first weight loads)
  const int NW = h.unw >> 8;
  const int r16 = lane & 15, kb = lane >> 4;

  int g0, g1;
  {
    const int ub = h.u_br & 0xFFFF, ur = h.u_br >> 16;
    const int U = h.unw & 0xFF;
    g0 = part_start(blockIdx.y, ub, ur) * U;
    g1 = part_start(blockIdx.y + 1, ub, ur) * U;
  }
  const uint32_t row_bytes = 32u * (uint32_t)h.G, d_tile_bytes = 256u * (uint32_t)((h.G + 7) >> 3);
  const int gw = g0 + wave * GS;                // first group of this wave
  const int vg = min(max(g1 - gw, 0), GS);      // its real groups
  const int64_t kw0 = (int64_t)gw * 128;        // first element of its K-range
  uint8_t* areg = lds + wave * (GS * M * 512);  // its operand bytes
  float* part = reinterpret_cast<float*>(lds + pq2_lds_part_offset(M, NW, GS));

  WgRows wr;
  if constexpr (MULTI) {
    wr = wg_rows<true>(a);
    args_in_one_batch(a, wr);
  } else {
    wr = wg_rows_head(h);
    wr.out = a.out;
    wr.N = a.N;
  }
  const int rb0 = wr.rb0, rb1 = wr.rb1;
  const int nrb = rb1 - rb0;

  // ---- activations first (the vector memory counter completes in order).
  // Lane l holds positions EPL*l .. EPL*l + EPL-1 of the wave's K-range: all
  // or half of one packed code word, in group l / LPG.
  const bool live = lane / LPG < vg;
  auto load_x = [&](int m, float (&v)[EPL]) {
    if (live) {
      const float4* src = reinterpret_cast<const float4*>(h.x + (int64_t)m * a.K + kw0) + (EPL / 4) * lane;
#pragma unroll
      for (int i = 0; i < EPL / 4; ++i) {
        const float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) v[i] = 0.f;
    }
  };
  float xv[MPRE][EPL];
#pragma unroll
  for (int m = 0; m < MPRE; ++m) load_x(m, xv[m]);

  const bool has_signs = h.signs != nullptr;
  uint32_t sw[EPL / 4];
#pragma unroll
  for (int i = 0; i < EPL / 4; ++i) sw[i] = 0u;
  if (live && has_signs) {
    if constexpr (EPL == 8) {
      const uint2 t = *reinterpret_cast<const uint2*>(h.signs + kw0 + 8 * lane);
      sw[0] = t.x; sw[1] = t.y;
    } else {
      const uint4 t = *reinterpret_cast<const uint4*>(h.signs + kw0 + 16 * lane);
      sw[0] = t.x; sw[1] = t.y; sw[2] = t.z; sw[3] = t.w;
    }
  }

  // ---- weight loads (pair q: groups 2q, 2q+1 of the wave)
  uint32_t qoff[GS / 2];
#pragma unroll
  for (int q = 0; q < GS / 2; ++q) {
    const int grp = 2 * q + (kb >> 1);
    qoff[q] = grp < vg ? (uint32_t)(gw + grp) * 512u + 32u * r16 + 16u * (kb & 1) : kOutOfRange;
  }
  // scales of row r16, group gw: chunk gw / 8 of the tile, row r16, slot gw % 8
  const uint32_t doff = (uint32_t)(gw >> 3) * 256u + (uint32_t)r16 * 16u + (uint32_t)(gw & 7) * 2u;
  using WB = WBuf<GS>;
  const int64_t wrow0 = (int64_t)rb0 * kRB;
  // codes: the workgroup's whole 16-row tiles (rows past N are zero padding)
  const BufRsrc rq = make_rsrc(wr.qs + wrow0 * row_bytes, (uint32_t)nrb * kRB * row_bytes);
  // scales: the workgroup's whole 16-row tiles of the scale plane (padding is zero)
  const BufRsrc rd = make_rsrc(wr.dpl + (int64_t)rb0 * d_tile_bytes, (uint32_t)nrb * d_tile_bytes);
  // this lane's row of block j, relative to the first block: inside the
  // workgroup's rows or loaded at kFarRows (zeros, no memory touched)
  const int rlo = wr.r0 - rb0 * kRB, rhi = wr.r1 - rb0 * kRB;
  auto issue = [&](int j, WB& b) {
    const int rl = j * kRB + r16;
    const bool mine = rl >= rlo && rl < rhi;
    const uint32_t ro = mine ? (uint32_t)j * (kRB * row_bytes) : kFarRows;
    const uint32_t rod = mine ? (uint32_t)j * d_tile_bytes : kFarRows;
    issue_row_block<GS, DALIGN>(b, rq, rd, qoff, doff, gw, r16, ro, rod);
  };
  // Only the first row block is loaded before the prologue.  A wave stalls at a
  // load it cannot issue while the compute unit's memory pipeline is full, and
  // a stalled wave does no arithmetic; with all D blocks issued here the waves
  // sat through the fetch and rotated x only afterwards.
  auto run = [&](auto early_tag) {
  // EARLY: all D row blocks before the prologue (see kEarlyWave)
  constexpr bool EARLY = decltype(early_tag)::value;
  // A raised wave priority through the prologue lets a wave that is still
  // rotating x issue ahead of waves already waiting on their loads; measured
  // 2% faster at 10240 x 5120 (the level, 1 to 3, made no difference).
  __builtin_amdgcn_s_setprio(1);
  WB wb[D];
  issue(0, wb[0]);
  if constexpr (EARLY) {
#pragma unroll
    for (int i = 1; i < D; ++i) issue(i, wb[i]);
  }

  // ---- per-wave prologue: rotation, per-group range scale, e5m2 terms
  float gsc[TILES][GS];  // 2^-e of (activation row 4*tile + kb, group)
  int sa[GS];            // ONE: E8M0 byte of 2^-e per group
#pragma unroll
  for (int g = 0; g < GS; ++g) sa[g] = 127;
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int g = 0; g < GS; ++g) gsc[t][g] = 0.f;
  {
    const int pw = (lane / C::LPW) & 7;              // packed word in the group
    const int half = lane % C::LPW;                  // which half of it (EPL = 8)
    const int kb16 = (0x76325410 >> (4 * pw)) & 15;  // {0,1,4,5,2,3,6,7}[pw]
    // MFMA operand position of the word: even positions of the word become
    // operand bytes 0..7, odd ones 8..15; a half word owns bytes 4*half + {0..3, 8..11}
    uint8_t* dst0 = areg + (lane / LPG) * M * 512 + (kb16 & 3) * 32 + (kb16 >> 2) * 16 + 4 * half;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v[EPL];
      if (m < MPRE) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) v[i] = xv[m < MPRE ? m : 0][i];
      } else {
        load_x(m, v);
      }
      if (has_signs) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const uint32_t neg = (sw[j >> 2] >> (8 * (j & 3) + 7)) & 1u;  // int8 sign bit
          v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (neg << 31));
        }
      }
      rotate<C::LOG_EPL>(v, a.log2n);
      // range scale of this lane's 128-group
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) mx = fmaxf(mx, fabsf(v[i]));
      mx = group_max<LPG>(mx);
      const int e = range_exponent(mx * a.inv_sqrt_n);
      // (the sign of this lane's quad butterflies rides on the scale)
      const float sc = ldexpf(a.inv_sqrt_n, e) * quad_stage_sign<C::LOG_EPL>(a.log2n);
      float r[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) r[i] = v[i] = v[i] * sc;
      // four e5m2 terms: t_k = e5m2(residual), residual -= t_k
      // bytes 0, 1 (term_lo) or 2, 3 (term_hi) of w
      auto term_lo = [&](int i0, int i1, int w) {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(r[i0], r[i1], w, false);
        const f32x2 back = __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
        r[i0] -= back.x;
        r[i1] -= back.y;
        return w;
      };
      auto term_hi = [&](int i0, int i1, int w) {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(r[i0], r[i1], w, true);
        const f32x2 back = __builtin_amdgcn_cvt_pk_f32_bf8(w, true);
        r[i0] -= back.x;
        r[i1] -= back.y;
        return w;
      };
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint8_t* dst = dst0 + (m * 4 + t) * 128;
        if constexpr (EPL == 8) {
          const int we = term_hi(4, 6, term_lo(0, 2, 0));
          const int wo = term_hi(5, 7, term_lo(1, 3, 0));
          if (live) {
            *reinterpret_cast<uint32_t*>(dst) = (uint32_t)we;
            *reinterpret_cast<uint32_t*>(dst + 8) = (uint32_t)wo;
          }
        } else {
          constexpr int P[16] = {0, 2, 4, 6, 8, 10, 12, 14, 1, 3, 5, 7, 9, 11, 13, 15};
          uint32_t tw[4];
#pragma unroll
          for (int dq = 0; dq < 4; ++dq) {
            tw[dq] = (uint32_t)term_hi(P[4 * dq + 2], P[4 * dq + 3], term_lo(P[4 * dq], P[4 * dq + 1], 0));
          }
          if (live) *reinterpret_cast<uint4*>(dst) = make_uint4(tw[0], tw[1], tw[2], tw[3]);
        }
      }
      // the lanes whose outputs belong to activation row m take 2^-e of every
      // group from the group's first lane
      const float inv = ldexpf(1.f, -e);
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        if constexpr (ONE) {
          if (g < vg) sa[g] = 127 - __builtin_amdgcn_readlane(e, LPG * g);
        } else {
          const float ig = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv), LPG * g));
#pragma unroll
          for (int t = 0; t < TILES; ++t)
            if (4 * t + kb == m && g < vg) gsc[t][g] = ig;
        }
      }
    }
  }
  // the other row blocks in flight (kept here by the scheduling barriers)
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!EARLY) {
#pragma unroll
    for (int i = 1; i < D; ++i) issue(i, wb[i]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // Lanes of rows past M and of groups past the slice read 32 zero bytes
  // (every wave stores the same zeros).  The operand bytes were written by
  // other lanes of this wave; LDS instructions of a wave complete in order, so
  // only the compiler must not move the reads above the writes.
  uint8_t* zeros = lds + pq2_lds_zero_offset(M, NW, GS);
  if (lane < 2) *reinterpret_cast<uint4*>(zeros + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
  // the output's address and row count in scalar registers now (left to the
  // compiler, their load from the argument block came after the final
  // barrier, on the critical path)
  asm volatile("" ::"s"(wr.out), "s"(wr.N));
  if constexpr (ONE) {
    // zeros in the partial slots of waves past NW: the sums need no mask
    if (wave == 0)
      for (int c = lane; c < 2 * RBR * kRB; c += 64)
        for (int w = NW; w < NWP; ++w) part[c * NWP + w] = 0.f;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int aop[TILES][GS][8];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    // activation row and term of this lane's operand row
    const int ma = ONE ? ((r16 & 3) == 0 ? 0 : M) : 4 * t + (r16 >> 2);
    const int tm = ONE ? r16 >> 2 : r16 & 3;
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const uint8_t* src = ma < M && g < vg ? areg + ((g * M + ma) * 4 + tm) * 128 + kb * 32 : zeros;
      const uint4* p = reinterpret_cast<const uint4*>(src);
      const uint4 p0 = p[0], p1 = p[1];
      aop[t][g][0] = p0.x; aop[t][g][1] = p0.y; aop[t][g][2] = p0.z; aop[t][g][3] = p0.w;
      aop[t][g][4] = p1.x; aop[t][g][5] = p1.y; aop[t][g][6] = p1.z; aop[t][g][7] = p1.w;
    }
  }

  // ---- main loop over row blocks
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const WB& b, int j) {
    uint2 wq[GS];
#pragma unroll
    for (int q = 0; q < GS / 2; ++q) pair_to_operands(b.q[q], wq[2 * q], wq[2 * q + 1]);
    // groups past the slice (g >= vg) read some other finite scale, or the
    // zero padding; their 2^-e and X are zero, so they add nothing
    float dg[GS];
#pragma unroll
    for (int g = 0; g < GS; ++g) dg[g] = f16_bits_to_f32((b.d[g >> 1] >> (16 * (g & 1))) & 0xFFFFu);
    f32x4 Y[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) Y[t] = zero;
    // Blocks of four groups.  The accumulators are read only after a delay
    // that is tied to them as asm operands: the compiler's wait-state count
    // for this mixed e5m2 x fp4 MFMA was measured to be too short on gfx950,
    // and the B registers stay untouched until the delay has passed.
#pragma unroll
    for (int h = 0; h < GS / 4; ++h) {
      i32x8 Bq[4];
      f32x4 acc[TILES][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t e0, o0, e1, o1;
        ternary_fp4(wq[4 * h + u].x, e0, o0);
        ternary_fp4(wq[4 * h + u].y, e1, o1);
        Bq[u] = (i32x8){(int)e0, (int)o0, (int)e1, (int)o1, 0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
          const int g = 4 * h + u;
          const i32x8 A = {aop[t][g][0], aop[t][g][1], aop[t][g][2], aop[t][g][3],
                           aop[t][g][4], aop[t][g][5], aop[t][g][6], aop[t][g][7]};
          acc[t][u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bq[u], zero, 1, 4, 0, sa[g], 0, 127);
        }
      static_assert(TILES <= 2, "the delay below lists the accumulators");
      if constexpr (TILES == 1) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3])
                     : "v"(Bq[0].lo), "v"(Bq[1].lo), "v"(Bq[2].lo), "v"(Bq[3].lo));
      } else {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]),
                       "+v"(acc[TILES - 1][0]), "+v"(acc[TILES - 1][1]), "+v"(acc[TILES - 1][2]),
                       "+v"(acc[TILES - 1][3])
                     : "v"(Bq[0].lo), "v"(Bq[1].lo), "v"(Bq[2].lo), "v"(Bq[3].lo));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
          const int g = 4 * h + u;
          if constexpr (ONE) {
            Y[0][0] = fmaf(dg[g], acc[0][u][0], Y[0][0]);
          } else {
            const float ds = dg[g] * gsc[t][g];
#pragma unroll
            for (int i = 0; i < 4; ++i) Y[t][i] = fmaf(ds, acc[t][u][i], Y[t][i]);
          }
        }
    }
    if constexpr (ONE) {
      // lane block kb holds term kb: the four added across the wave
      // ((kb 0 + kb 2) + (kb 1 + kb 3), the same bits in every lane of a row)
      float t = Y[0][0];
      t += xor_lane<32>(t);
      t += xor_lane<16>(t);
      if (kb == 0) part[((((j / RBR) & 1) * RBR + j % RBR) * kRB + r16) * NWP + wave] = 2.f * t;
    } else {
      float* pw = part + ((((j / RBR) & 1) * NW + wave) * RBR + j % RBR) * M * KS * kRB;
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int mo = 4 * t + kb;
        if (mo < M) pw[mo * kRB + r16] = 2.f * ((Y[t][0] + Y[t][1]) + (Y[t][2] + Y[t][3]));
      }
    }
  };
  auto reduce = [&](int round) {
    if constexpr (ONE) reduce_round_one<NWP>(wr, part, RBR, rb0, nrb, round, blockIdx.y);
    else reduce_round(wr, part, NW, RBR, M, KS, rb0, nrb, round, blockIdx.y);
  };

  if constexpr (FEW) {
    // every row block is already in flight: no further loads
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (i < nrb) compute(wb[i], i);
    if constexpr (ONE) {
      // the final sums' operands and destinations, ready before the barrier
      // (at most D row blocks: threads [0, 16 D) hold one output each)
      const int jr = threadIdx.x / kRB;
      const int row = (rb0 + jr) * kRB + (int)(threadIdx.x % kRB);
      const bool ok = jr < nrb && row >= wr.r0 && row < wr.r1;
      float* dst = wr.out + (int64_t)blockIdx.y * wr.N + row;
      const float* src = part + threadIdx.x * NWP;
      __syncthreads();
      if (ok) *dst = sum_slots<NWP>(src);
    } else {
      __syncthreads();
      reduce(0);
    }
    return;
  }
  for (int j0 = 0; j0 < nrb; j0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int j = j0 + i;
      if (j < nrb) compute(wb[i], j);
      issue(j + D, wb[i]);
      if (j < nrb && (j % RBR == RBR - 1 || j == nrb - 1)) {
        __syncthreads();
        reduce(j / RBR);
      }
    }
  }
  };
  if constexpr (FEW) {
    if (wave >= kEarlyWave) run(std::true_type{});
    else run(std::false_type{});
  } else {
    run(std::false_type{});
  }
}


// ---------------------------------------------------------------------------
// Q8_0
//
// The int8 weights are the B operand of v_mfma_i32_16x16x32_i8 as loaded.  x'
// is scaled per activation row (over the workgroup's K slice) by a power of two
// 2^s that puts its largest magnitude in [2^29, 2^30), rounded to an integer
// I = rne(x' 2^s) (within 1/2, i.e. 2^-30 of the row's largest magnitude), and
// written as four signed base-256 digits, most significant first:
// I = sum_t d_t 256^(3-t) with every d_t in [-128, 127].  J = I + 0x80808080 is
// non-negative and its bytes are d_t + 128 (base-256 digits of J), so the
// digits are J's bytes with their top bit flipped.  Operand row 4t + m holds
// digit t of activation row m, so lane block kb ends with digit kb of every
// row; each group's integer sum (below 32*127*128 in magnitude) converts to fp32
// exactly and is scaled by the group's fp16 d.  The digit weight 256^(3-kb)
// and 2^-s are applied once per row block, and the four lane blocks' partials
// are added by the LDS reduction in a fixed order.

// Groups of 32 per wave: 16 (two chunks of scales) up to four activation
// rows; 8 for the bf16 kernel of five to eight rows, whose waves then fit 168
// VGPRs, so that a workgroup holds 10 waves (two K slices at K=5120) instead
// of 5 of 16 groups (M=8: 26.2 -> 22.8 us; its LDS, the staged rows of x,
// leaves room for one workgroup per compute unit).  Row blocks of weight
// loads in flight: two for one activation row, one for two to four (their
// digit operands take the registers), two again for five to eight.
__host__ __device__ constexpr int q8_rbr(int M) { return M == 1 ? 8 : 2; }  // row blocks per reduction round
__host__ __device__ constexpr int q8_maxw(int) { return 12; }
__host__ __device__ constexpr int q8_gs(int M) { return M > 4 ? 8 : 16; }
template <int M>
struct Q8Cfg {
  static constexpr int GS = q8_gs(M);
  static constexpr int D = M == 1 || M > 4 ? 2 : 1;
  static constexpr int RBR = q8_rbr(M);
  static constexpr int MAXW = q8_maxw(M);
};

// LDS bytes: x' staged as fp32 [M][NW*GS*32] and rewritten in place as digits
// (each 8-element chunk: [4 digits][8 bytes]), the slice maxima [M][NW], the
// partials [2][NW][RBR][M][4 lane blocks][16] floats, then 16 zero bytes
__host__ __device__ inline int q8_lds_max_offset(int M, int NW, int GS) { return M * NW * GS * 32 * 4; }
__host__ __device__ inline int q8_lds_part_offset(int M, int NW, int GS) {
  return q8_lds_max_offset(M, NW, GS) + (M * NW * 4 + 15) / 16 * 16;
}
__host__ __device__ inline int q8_lds_zero_offset(int M, int NW, int GS) {
  return q8_lds_part_offset(M, NW, GS) + 2 * NW * q8_rbr(M) * M * 4 * kRB * 4;
}
__host__ __device__ inline int q8_lds_bytes(int M, int NW, int GS) { return q8_lds_zero_offset(M, NW, GS) + 16; }

// rotation stages with h >= 16 in LDS: butterflies on E = 2^L values at stride 16
template <int L>
__device__ void lds_stages_t(float* xs, int KRmax, int KR, int n, int M_) {
  constexpr int E = 1 << L;
  const int items = KR / E;
  for (int m = 0; m < M_; ++m) {
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
      float* p = xs + m * KRmax + (it >> 4) * n + (it & 15);
      float v[E];
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = p[16 * i];
#pragma unroll
      for (int st = 0; st < L; ++st) {
        const int h = 1 << st;
#pragma unroll
        for (int i = 0; i < E; ++i)
          if ((i & h) == 0) {
            const float p0 = v[i], p1 = v[i + h];
            v[i] = p0 + p1;
            v[i + h] = p0 - p1;
          }
      }
#pragma unroll
      for (int i = 0; i < E; ++i) p[16 * i] = v[i];
    }
  }
}
__device__ void lds_stages(float* xs, int KRmax, int KR, int log2n, int M_) {
  const int n = 1 << log2n;
  switch (log2n) {
    case 5: lds_stages_t<1>(xs, KRmax, KR, n, M_); break;
    case 6: lds_stages_t<2>(xs, KRmax, KR, n, M_); break;
    case 7: lds_stages_t<3>(xs, KRmax, KR, n, M_); break;
    case 8: lds_stages_t<4>(xs, KRmax, KR, n, M_); break;
    case 9: lds_stages_t<5>(xs, KRmax, KR, n, M_); break;
    default: lds_stages_t<6>(xs, KRmax, KR, n, M_); break;
  }
}

// maximum over the 64 lanes of a wave, every lane receiving it (v >= 0: the
// integer maximum of the bit patterns)
__device__ __forceinline__ float wave_max_nonneg(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, true));
  u = max(max((uint32_t)__builtin_amdgcn_readlane((int)u, 0), (uint32_t)__builtin_amdgcn_readlane((int)u, 16)),
          max((uint32_t)__builtin_amdgcn_readlane((int)u, 32), (uint32_t)__builtin_amdgcn_readlane((int)u, 48)));
  return __uint_as_float(u);
}

// exponent s that puts bound * 2^s in [2^29, 2^30), within [-126, 126] so that 2^s
// and 2^-s stay finite (0 for a zero, infinite or NaN bound)
__device__ __forceinline__ int digit_exponent(float bound) {
  const uint32_t ef = (__float_as_uint(bound) >> 23) & 0xFFu;
  if (!(bound > 0.f) || ef == 0xFFu) return 0;
  const int e = 29 - ((int)ef - 127);
  return e < -126 ? -126 : (e > 126 ? 126 : e);
}

// 4 x 4 byte transpose: out[k] = [j0.k, j1.k, j2.k, j3.k] (byte k of each word,
// in order), eight v_perm_b32
__device__ __forceinline__ void transpose_bytes(uint32_t j0, uint32_t j1, uint32_t j2, uint32_t j3,
                                                uint32_t (&out)[4]) {
  const uint32_t p_lo = __builtin_amdgcn_perm(j1, j0, 0x05010400u);  // [j0.0, j1.0, j0.1, j1.1]
  const uint32_t p_hi = __builtin_amdgcn_perm(j1, j0, 0x07030602u);  // [j0.2, j1.2, j0.3, j1.3]
  const uint32_t q_lo = __builtin_amdgcn_perm(j3, j2, 0x05010400u);
  const uint32_t q_hi = __builtin_amdgcn_perm(j3, j2, 0x07030602u);
  out[0] = __builtin_amdgcn_perm(q_lo, p_lo, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(q_lo, p_lo, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(q_hi, p_hi, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(q_hi, p_hi, 0x07060302u);
}

template <int M, bool DALIGN, bool MULTI>
__global__ __launch_bounds__(Q8Cfg<M>::MAXW * 64) void gemv_q8_kernel(GemvArgs a) {
  static_assert(M <= 4, "one operand tile: four digits of up to four activation rows");
  constexpr int GS = Q8Cfg<M>::GS, D = Q8Cfg<M>::D, RBR = Q8Cfg<M>::RBR;
  constexpr int TILES = (M + 3) / 4;
  extern __shared__ __align__(16) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NW = blockDim.x >> 6;
  const int r16 = lane & 15, kb = lane >> 4;

  int g0, g1;
  slice_groups(a, blockIdx.y, g0, g1);
  const int KR = (g1 - g0) * 32;
  const int64_t k0 = (int64_t)g0 * 32;
  const int gw = wave * GS;  // relative to g0
  const int vg = min(max(g1 - g0 - gw, 0), GS);
  const int KRmax = NW * GS * 32;
  float* xs = reinterpret_cast<float*>(lds);  // [M][KRmax]
  float* rmax = reinterpret_cast<float*>(lds + q8_lds_max_offset(M, NW, GS));  // [M][NW]
  float* part = reinterpret_cast<float*>(lds + q8_lds_part_offset(M, NW, GS));
  uint8_t* zeros = lds + q8_lds_zero_offset(M, NW, GS);

  const WgRows wr = wg_rows<MULTI>(a);
  args_in_one_batch(a, wr);
  const int rb0 = wr.rb0, rb1 = wr.rb1;
  const int nrb = rb1 - rb0;

  // ---- activation loads first.  A thread holds one 16-element unit of up to
  // MR rows: for two to four rows the threads of units [0, U16) take the
  // first MR rows and those of [U16, 2 U16) the rest (a slice has at most
  // half as many units as the workgroup has threads), so every thread works
  // on the prologue and none holds more than two rows.
  constexpr int RG = M >= 2 ? 2 : 1;      // row groups
  constexpr int MR = (M + RG - 1) / RG;   // rows per thread
  static_assert(GS * 32 / 16 * RG <= 64, "a wave's units of all row groups fit its lanes");
  const int U16 = KR >> 4;                // 16-element units per activation row
  const int rg = tid >= U16 ? 1 : 0;
  const int u = tid - rg * U16;           // the thread's unit
  const bool has_unit = tid < RG * U16;
  auto row_of = [&](int i) { return rg * MR + i; };
  auto load_row = [&](int m, float (&v)[16]) {
    if (has_unit && m < M) {
      const float4* src = reinterpret_cast<const float4*>(a.x + (int64_t)m * a.K + k0) + 4 * u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.f;
    }
  };
  float xv[MR][16];
  uint4 sg = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 0; i < MR; ++i) load_row(row_of(i), xv[i]);
  if (has_unit && a.signs) sg = *reinterpret_cast<const uint4*>(a.signs + k0 + 16 * u);

  // ---- weight loads (pair q: groups 2q, 2q+1 of the wave)
  uint32_t qoff[GS / 2];
#pragma unroll
  for (int q = 0; q < GS / 2; ++q) {
    const int grp = 2 * q + (kb >> 1);
    qoff[q] = grp < vg ? (uint32_t)(g0 + gw + grp) * 512u + 32u * r16 + 16u * (kb & 1) : kOutOfRange;
  }
  // scales of row r16, group gq = g0 + gw: chunk gq / 8 of the tile, row r16, slot gq % 8
  const int gq = g0 + gw;
  const uint32_t doff = (uint32_t)(gq >> 3) * 256u + (uint32_t)r16 * 16u + (uint32_t)(gq & 7) * 2u;
  using WB = WBuf<GS>;
  const int64_t wrow0 = (int64_t)rb0 * kRB;
  // codes: the workgroup's whole 16-row tiles (rows past N are zero padding)
  const BufRsrc rq = make_rsrc(wr.qs + wrow0 * a.row_bytes, (uint32_t)nrb * kRB * a.row_bytes);
  const BufRsrc rd = make_rsrc(wr.dpl + (int64_t)rb0 * a.d_tile_bytes, (uint32_t)nrb * a.d_tile_bytes);
  // this lane's row of block j, relative to the first block: inside the
  // workgroup's rows or loaded at kFarRows (zeros, no memory touched)
  const int rlo = wr.r0 - rb0 * kRB, rhi = wr.r1 - rb0 * kRB;
  auto issue = [&](int j, WB& b) {
    const int rl = j * kRB + r16;
    const bool mine = rl >= rlo && rl < rhi;
    const uint32_t ro = mine ? (uint32_t)j * (kRB * a.row_bytes) : kFarRows;
    const uint32_t rod = mine ? (uint32_t)j * a.d_tile_bytes : kFarRows;
    issue_row_block<GS, DALIGN>(b, rq, rd, qoff, doff, gq, r16, ro, rod);
  };

  // One row: only the first row block is requested before the prologue (a
  // wave stalls at a load it cannot issue while the memory pipeline is full,
  // and a stalled wave does no arithmetic); the rest after it.
  constexpr int DPRE = M == 1 ? 1 : D;
  WB wb[D];
#pragma unroll
  for (int i = 0; i < DPRE; ++i) issue(i, wb[i]);

  // ---- prologue: stage x (.) s in LDS, butterflies with stride < 16 in
  // registers, wider ones in LDS.  Without LDS stages each thread's values
  // are final in its registers, so their maxima are taken there (one LDS
  // pass and one barrier fewer).
  const bool reg_max = a.log2n <= 4;
  float mx[M];
#pragma unroll
  for (int m = 0; m < M; ++m) mx[m] = 0.f;
  float xr[MR][16];  // the thread's rows of x (.) s after the in-register stages
  {
    const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
    for (int ir = 0; ir < MR; ++ir) {
      const int m = row_of(ir);
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = xv[ir][i];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t neg = (sw[j >> 2] >> (8 * (j & 3) + 7)) & 1u;  // int8 sign bit
        v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (neg << 31));
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st < a.log2n) {
          const int h = 1 << st;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
              const float p0 = v[i], p1 = v[i + h];
              v[i] = p0 + p1;
              v[i + h] = p0 - p1;
            }
        }
      }
      // staged in LDS only for the rotation stages there (wider blocks);
      // otherwise the digits are made from these registers
      if (!reg_max && has_unit && m < M) {
        float4* dst = reinterpret_cast<float4*>(xs + m * KRmax) + 4 * u;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
      }
      float vm = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) vm = fmaxf(vm, fabsf(v[i]));  // (zeros past the slice)
#pragma unroll
      for (int mm = 0; mm < M; ++mm)
        if (mm == m) mx[mm] = vm;
#pragma unroll
      for (int i = 0; i < 16; ++i) xr[ir][i] = v[i];
    }
  }
  if (reg_max) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float w = wave_max_nonneg(mx[m]);
      if (lane == 0) rmax[m * NW + wave] = w;
    }
    if (tid < 4) reinterpret_cast<uint32_t*>(zeros)[tid] = 0u;
  }
  __syncthreads();
  if (!reg_max) {
    lds_stages(xs, KRmax, KR, a.log2n, M);
    __syncthreads();
  }

  // ---- digits: the slice's largest |x'| per row, then every 8-element chunk
  // of x' rewritten in place as its four digit planes
  const int nch = KR >> 3;
  if (!reg_max) {
#pragma unroll
    for (int m = 0; m < M; ++m) mx[m] = 0.f;
    for (int c = tid; c < nch; c += blockDim.x) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float4* src = reinterpret_cast<const float4*>(xs + m * KRmax + 8 * c);
        const float4 f0 = src[0], f1 = src[1];
        mx[m] = fmaxf(mx[m], fmaxf(fmaxf(fmaxf(fabsf(f0.x), fabsf(f0.y)), fmaxf(fabsf(f0.z), fabsf(f0.w))),
                                   fmaxf(fmaxf(fabsf(f1.x), fabsf(f1.y)), fmaxf(fabsf(f1.z), fabsf(f1.w)))));
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float w = wave_max_nonneg(mx[m]);
      if (lane == 0) rmax[m * NW + wave] = w;
    }
    if (tid < 4) reinterpret_cast<uint32_t*>(zeros)[tid] = 0u;
    __syncthreads();
  }
  float cs[M];   // inv_sqrt_n * 2^s: x' 2^s = staged value * cs
  float ysc[M];  // 2^-s
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float r = 0.f;
    for (int w = 0; w < NW; ++w) r = fmaxf(r, rmax[m * NW + w]);
    const int e = digit_exponent(r * a.inv_sqrt_n);
    cs[m] = ldexpf(a.inv_sqrt_n, e);
    ysc[m] = ldexpf(1.f, -e);
  }
  {
    constexpr uint32_t kBias = 0x80808080u;
    // one 8-element chunk of row m: its four digit planes at ptr
    auto digits = [&](const float (&v)[8], float c, float4* ptr) {
      uint32_t J[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) J[i] = (uint32_t)(int)__builtin_rintf(v[i] * c) + kBias;
      // plane t (digit t) is byte 3 - t of each J, top bit flipped
      uint32_t lo[4], hi[4];
      transpose_bytes(J[0], J[1], J[2], J[3], lo);
      transpose_bytes(J[4], J[5], J[6], J[7], hi);
      ptr[0] = __builtin_bit_cast(float4, make_uint4(lo[3] ^ kBias, hi[3] ^ kBias, lo[2] ^ kBias, hi[2] ^ kBias));
      ptr[1] = __builtin_bit_cast(float4, make_uint4(lo[1] ^ kBias, hi[1] ^ kBias, lo[0] ^ kBias, hi[0] ^ kBias));
    };
    if (reg_max) {
      // from the thread's registers: its unit's two chunks of each of its rows
      if (has_unit) {
#pragma unroll
        for (int ir = 0; ir < MR; ++ir) {
          const int m = row_of(ir);
          float c = 0.f;
#pragma unroll
          for (int mm = 0; mm < M; ++mm)
            if (mm == m) c = cs[mm];
          if (m < M) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float v[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) v[i] = xr[ir][8 * h + i];
              digits(v, c, reinterpret_cast<float4*>(xs + m * KRmax + 16 * u + 8 * h));
            }
          }
        }
      }
    } else {
      // in place, from the staged and rotated rows
      for (int c = tid; c < nch; c += blockDim.x) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float4* ptr = reinterpret_cast<float4*>(xs + m * KRmax + 8 * c);
          const float4 f0 = ptr[0], f1 = ptr[1];
          const float v[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
          digits(v, cs[m], ptr);
        }
      }
    }
  }
  __syncthreads();

  if constexpr (DPRE < D) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = DPRE; i < D; ++i) issue(i, wb[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- operand: lane (r16, kb) holds digit r16 / 4 of activation row
  // 4 * tile + r16 % 4 at the 8 positions that operand block kb covers (the
  // weight operand's order: bytes {0, 16, 8, 24}[kb] + 0..7 of each group)
  long aop[TILES][GS];
  float pscale[TILES][4];  // 2^-s * 256^(3 - kb) of the lane's output rows
  {
    const int dt = r16 >> 2;
    const int base = ((kb & 1) << 4) | ((kb & 2) << 2);  // {0, 16, 8, 24}[kb]
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int ma = 4 * t + (r16 & 3);
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        const int pos = (gw + g) * 32 + base;
        const uint8_t* src =
            ma < M && g < vg ? reinterpret_cast<const uint8_t*>(xs + (ma < M ? ma : 0) * KRmax + pos) + 8 * dt : zeros;
        aop[t][g] = *reinterpret_cast<const long*>(src);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pscale[t][i] = 4 * t + i < M ? ldexpf(ysc[4 * t + i < M ? 4 * t + i : 0], 8 * (3 - kb)) : 0.f;
    }
  }

  // ---- main loop over row blocks.  Two to four rows (one row block in
  // flight): each part of a row block's buffer is refilled with row block
  // j + D as soon as it has been read, so the wave's next loads go out while
  // it computes; with the whole block issued after the compute the memory sat
  // idle while every wave computed.  One row keeps two whole blocks in flight.
  constexpr bool ROLL = M > 1;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 izero = {0, 0, 0, 0};
  auto compute = [&](WB& b, int j) {
    const int jn = j + D;
    const int rln = jn * kRB + r16;
    const bool mine = rln >= rlo && rln < rhi;
    const uint32_t ro = mine ? (uint32_t)jn * (kRB * a.row_bytes) : kFarRows;
    const uint32_t rod = mine ? (uint32_t)jn * a.d_tile_bytes : kFarRows;
    float Y[TILES][4];
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[t][i] = 0.f;
#pragma unroll
    for (int q = 0; q < GS / 2; ++q) {
      uint2 wq[2];
      pair_to_operands(b.q[q], wq[0], wq[1]);
      // groups past the slice have zero operands; their scale is some other
      // finite one, or zero past the plane
      float dpair[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) dpair[h] = f16_bits_to_f32((b.d[q] >> (16 * h)) & 0xFFFFu);
      if constexpr (ROLL) {
        issue_codes<GS>(b, q, rq, qoff[q], ro);
        if (DALIGN ? q % 4 == 3 : true) issue_scales<GS, DALIGN>(b, DALIGN ? q / 4 : q, rd, doff, gq, r16, rod);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * q + h;
        const float dd = dpair[h];
        const long bq = (long)(((uint64_t)wq[h].y << 32) | wq[h].x);
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
          const i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[t][g], bq, izero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * t + i < M) Y[t][i] = fmaf(dd, (float)acc[i], Y[t][i]);
        }
      }
    }
    float* pw = part + ((((j / RBR) & 1) * NW + wave) * RBR + j % RBR) * M * 4 * kRB;
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * t + i < M) pw[((4 * t + i) * 4 + kb) * kRB + r16] = Y[t][i] * pscale[t][i];
  };

  for (int j0 = 0; j0 < nrb; j0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int j = j0 + i;
      if (j < nrb) compute(wb[i], j);  // (ROLL: its loads of row block j + D included)
      if constexpr (!ROLL) issue(j + D, wb[i]);
      if (j < nrb && (j % RBR == RBR - 1 || j == nrb - 1)) {
        __syncthreads();
        reduce_round(wr, part, NW, RBR, M, 4, rb0, nrb, j / RBR, blockIdx.y);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Q8_0, five to eight activation rows: the int8 digits would need two operand
// tiles (two MFMAs per group); here each int8 weight converts to bf16 exactly
// and x enters as bf16 hi + lo parts (2^-17 relative), so one
// v_mfma_f32_16x16x32_bf16 covers 16 weight rows x one 32-group for all 8
// rows.  Lane (i, kb) of the operand holds activation row i/2 (hi part for
// even i, lo for odd i).

// LDS bytes: staged activations f32 [M][NW*GS*32], then the partials
// [2][NW][RBR][M][16] floats
__host__ __device__ inline int q8b_lds_part_offset(int M, int NW, int GS) { return M * NW * GS * 32 * 4; }
__host__ __device__ inline int q8b_lds_bytes(int M, int NW, int GS) {
  return q8b_lds_part_offset(M, NW, GS) + 2 * NW * q8_rbr(M) * M * kRB * 4;
}

template <int M, bool DALIGN, bool MULTI>
__global__ __launch_bounds__(Q8Cfg<M>::MAXW * 64) void gemv_q8_bf16_kernel(GemvArgs a) {
  constexpr int GS = Q8Cfg<M>::GS, D = Q8Cfg<M>::D, RBR = Q8Cfg<M>::RBR;
  extern __shared__ __align__(16) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NW = blockDim.x >> 6;
  const int r16 = lane & 15, kb = lane >> 4;

  int g0, g1;
  slice_groups(a, blockIdx.y, g0, g1);
  const int KR = (g1 - g0) * 32;
  const int64_t k0 = (int64_t)g0 * 32;
  const int gw = wave * GS;  // relative to g0
  const int vg = min(max(g1 - g0 - gw, 0), GS);
  const int KRmax = NW * GS * 32;
  float* xs = reinterpret_cast<float*>(lds);  // [M][KRmax]
  float* part = reinterpret_cast<float*>(lds + q8b_lds_part_offset(M, NW, GS));

  const WgRows wr = wg_rows<MULTI>(a);
  args_in_one_batch(a, wr);
  const int rb0 = wr.rb0, rb1 = wr.rb1;
  const int nrb = rb1 - rb0;

  // ---- activation loads first (rows past the first four after the weight
  // loads, to bound the registers held)
  constexpr int MPRE = M < 4 ? M : 4;
  const int U16 = KR >> 4;  // 16-element units per activation row (<= threads)
  const bool has_unit = tid < U16;
  auto load_row = [&](int m, float (&v)[16]) {
    if (has_unit) {
      const float4* src = reinterpret_cast<const float4*>(a.x + (int64_t)m * a.K + k0) + 4 * tid;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.f;
    }
  };
  float xv[MPRE][16];
  uint4 sg = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int m = 0; m < MPRE; ++m) load_row(m, xv[m]);
  if (has_unit && a.signs) sg = *reinterpret_cast<const uint4*>(a.signs + k0 + 16 * tid);

  // ---- weight loads (pair q: groups 2q, 2q+1 of the wave)
  uint32_t qoff[GS / 2];
#pragma unroll
  for (int q = 0; q < GS / 2; ++q) {
    const int grp = 2 * q + (kb >> 1);
    qoff[q] = grp < vg ? (uint32_t)(g0 + gw + grp) * 512u + 32u * r16 + 16u * (kb & 1) : kOutOfRange;
  }
  // scales of row r16, group gq = g0 + gw: chunk gq / 8 of the tile, row r16, slot gq % 8
  const int gq = g0 + gw;
  const uint32_t doff = (uint32_t)(gq >> 3) * 256u + (uint32_t)r16 * 16u + (uint32_t)(gq & 7) * 2u;
  using WB = WBuf<GS>;
  const int64_t wrow0 = (int64_t)rb0 * kRB;
  // codes: the workgroup's whole 16-row tiles (rows past N are zero padding)
  const BufRsrc rq = make_rsrc(wr.qs + wrow0 * a.row_bytes, (uint32_t)nrb * kRB * a.row_bytes);
  const BufRsrc rd = make_rsrc(wr.dpl + (int64_t)rb0 * a.d_tile_bytes, (uint32_t)nrb * a.d_tile_bytes);
  // this lane's row of block j, relative to the first block: inside the
  // workgroup's rows or loaded at kFarRows (zeros, no memory touched)
  const int rlo = wr.r0 - rb0 * kRB, rhi = wr.r1 - rb0 * kRB;
  auto issue = [&](int j, WB& b) {
    const int rl = j * kRB + r16;
    const bool mine = rl >= rlo && rl < rhi;
    const uint32_t ro = mine ? (uint32_t)j * (kRB * a.row_bytes) : kFarRows;
    const uint32_t rod = mine ? (uint32_t)j * a.d_tile_bytes : kFarRows;
    issue_row_block<GS, DALIGN>(b, rq, rd, qoff, doff, gq, r16, ro, rod);
  };

  WB wb[D];
#pragma unroll
  for (int i = 0; i < D; ++i) issue(i, wb[i]);

  // ---- prologue: stage x (.) s in LDS, butterflies with stride < 16 in
  // registers, wider ones in LDS
  {
    const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v[16];
      if (m < MPRE) {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = xv[m < MPRE ? m : 0][i];
      } else {
        load_row(m, v);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t neg = (sw[j >> 2] >> (8 * (j & 3) + 7)) & 1u;  // int8 sign bit
        v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (neg << 31));
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st < a.log2n) {
          const int h = 1 << st;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
              const float p0 = v[i], p1 = v[i + h];
              v[i] = p0 + p1;
              v[i + h] = p0 - p1;
            }
        }
      }
      if (has_unit) {
        float4* dst = reinterpret_cast<float4*>(xs + m * KRmax) + 4 * tid;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
      }
    }
  }
  __syncthreads();
  if (a.log2n > 4) {
    lds_stages(xs, KRmax, KR, a.log2n, M);
    __syncthreads();
  }

  // ---- operand: lane (i, kb) holds activation row i/2 (hi part for even i,
  // lo for odd i) at the 8 positions that operand block kb covers
  int aop[GS][4];
  {
    const int ma = r16 >> 1;
    const bool lo_part = r16 & 1;
    const int base = ((kb & 1) << 4) | ((kb & 2) << 2);  // {0, 16, 8, 24}[kb]
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      if (ma < M && g < vg) {
        const float4* p = reinterpret_cast<const float4*>(xs + ma * KRmax + (gw + g) * 32 + base);
        const float4 f0 = p[0], f1 = p[1];
        const float v[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e0 = v[2 * i] * a.inv_sqrt_n, e1 = v[2 * i + 1] * a.inv_sqrt_n;
          const uint32_t hh = pack_bf16x2(e0, e1);
          const uint32_t ll = pack_bf16x2(e0 - bf16_bits_to_f32(hh & 0xFFFFu), e1 - bf16_bits_to_f32(hh >> 16));
          aop[g][i] = (int)(lo_part ? ll : hh);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) aop[g][i] = 0;
      }
    }
  }

  // ---- main loop over row blocks
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const WB& b, int j) {
    f32x4 Y = zero;
#pragma unroll
    for (int q = 0; q < GS / 2; ++q) {
      uint2 wq[2];
      pair_to_operands(b.q[q], wq[0], wq[1]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * q + h;
        const float dd = f16_bits_to_f32((b.d[g >> 1] >> (16 * (g & 1))) & 0xFFFFu);
        const float dg = g < vg ? dd : 0.f;
        const uint32_t w0 = wq[h].x, w1 = wq[h].y;
        const uint4 bq = make_uint4(bf16_pair(i8_as_f32bits(w0, 0), i8_as_f32bits(w0, 1)),
                                    bf16_pair(i8_as_f32bits(w0, 2), i8_as_f32bits(w0, 3)),
                                    bf16_pair(i8_as_f32bits(w1, 0), i8_as_f32bits(w1, 1)),
                                    bf16_pair(i8_as_f32bits(w1, 2), i8_as_f32bits(w1, 3)));
        const uint4 aq = make_uint4((uint32_t)aop[g][0], (uint32_t)aop[g][1], (uint32_t)aop[g][2],
                                    (uint32_t)aop[g][3]);
        const f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, aq), __builtin_bit_cast(bf16x8, bq), zero, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = fmaf(dg, acc[i], Y[i]);
      }
    }
    float* pw = part + ((((j / RBR) & 1) * NW + wave) * RBR + j % RBR) * M * kRB;
    const int m0 = 2 * kb;
    if (m0 < M) pw[m0 * kRB + r16] = Y[0] + Y[1];
    if (m0 + 1 < M) pw[(m0 + 1) * kRB + r16] = Y[2] + Y[3];
  };

  for (int j0 = 0; j0 < nrb; j0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int j = j0 + i;
      if (j < nrb) compute(wb[i], j);
      issue(j + D, wb[i]);
      if (j < nrb && (j % RBR == RBR - 1 || j == nrb - 1)) {
        __syncthreads();
        reduce_round(wr, part, NW, RBR, M, 1, rb0, nrb, j / RBR, blockIdx.y);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Loads-only twin of the GEMV kernels (a measurement instrument): the same
// grid, workgroup shape, activation loads and weight loads per wave
// (issue_row_block with the same offsets and the same number of row blocks in
// flight), every loaded word XOR-ed into one register; no rotation, no matrix
// products, no reduction.  sink[0] is written only if the XOR equals an
// unlikely constant, so that no load can be dropped.

// launch bounds of the GEMV the twin stands for (its register budget: with
// 1024 threads the 8-group twin spilled its in-flight row blocks)
template <bool PQ2, int GS, int D, bool DALIGN>
__global__ __launch_bounds__((PQ2 ? Pq2Cfg<2 * GS>::MAXW : q8_maxw(1)) * 64) void gemv_loads_twin_kernel(GemvArgs a, int M, uint32_t* sink) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kb = lane >> 4;
  int g0, g1;
  slice_groups(a, blockIdx.y, g0, g1);
  const int gw = g0 + wave * GS;            // first group of this wave
  const int vg = min(max(g1 - gw, 0), GS);  // its real groups
  const WgRows wr = wg_rows<false>(a);
  args_in_one_batch(a, wr);
  const int rb0 = wr.rb0, nrb = wr.rb1 - wr.rb0;
  uint32_t acc = 0;
  // activations: the PQ2_0 kernel's lanes hold 2 GS consecutive elements of
  // the wave's K-range, the Q8_0 kernel's threads 16 of the workgroup's slice
  if constexpr (PQ2) {
    constexpr int EPL = 2 * GS;
    if (lane / (128 / EPL) < vg)
      for (int m = 0; m < M; ++m) {
        const uint4* src = reinterpret_cast<const uint4*>(a.x + (int64_t)m * a.K + (int64_t)gw * 128) + (EPL / 4) * lane;
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) {
          const uint4 f = src[i];
          acc ^= f.x ^ f.y ^ f.z ^ f.w;
        }
      }
  } else {
    if (tid < ((g1 - g0) * 32) >> 4)
      for (int m = 0; m < M; ++m) {
        const uint4* src = reinterpret_cast<const uint4*>(a.x + (int64_t)m * a.K + (int64_t)g0 * 32) + 4 * tid;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 f = src[i];
          acc ^= f.x ^ f.y ^ f.z ^ f.w;
        }
      }
  }
  uint32_t qoff[GS / 2];
#pragma unroll
  for (int q = 0; q < GS / 2; ++q) {
    const int grp = 2 * q + (kb >> 1);
    qoff[q] = grp < vg ? (uint32_t)(gw + grp) * 512u + 32u * r16 + 16u * (kb & 1) : kOutOfRange;
  }
  const uint32_t doff = (uint32_t)(gw >> 3) * 256u + (uint32_t)r16 * 16u + (uint32_t)(gw & 7) * 2u;
  const BufRsrc rq = make_rsrc(wr.qs + (int64_t)rb0 * kRB * a.row_bytes, (uint32_t)nrb * kRB * a.row_bytes);
  const BufRsrc rd = make_rsrc(wr.dpl + (int64_t)rb0 * a.d_tile_bytes, (uint32_t)nrb * a.d_tile_bytes);
  const int rlo = wr.r0 - rb0 * kRB, rhi = wr.r1 - rb0 * kRB;
  auto issue = [&](int j, WBuf<GS>& b) {
    const int rl = j * kRB + r16;
    const bool mine = rl >= rlo && rl < rhi;
    const uint32_t ro = mine ? (uint32_t)j * (kRB * a.row_bytes) : kFarRows;
    const uint32_t rod = mine ? (uint32_t)j * a.d_tile_bytes : kFarRows;
    issue_row_block<GS, DALIGN>(b, rq, rd, qoff, doff, gw, r16, ro, rod);
  };
  WBuf<GS> wb[D];
#pragma unroll
  for (int i = 0; i < D; ++i) issue(i, wb[i]);
  if (PQ2 && nrb <= D) {
    // as the PQ2_0 GEMV: every row block is in flight, no further loads
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (i < nrb) {
#pragma unroll
        for (int q = 0; q < GS / 2; ++q) acc ^= wb[i].q[q].x ^ wb[i].q[q].y ^ wb[i].q[q].z ^ wb[i].q[q].w ^ wb[i].d[q];
      }
    if (acc == 0x9E3779B9u) sink[0] = acc;
    return;
  }
  for (int j0 = 0; j0 < nrb; j0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int j = j0 + i;
      if (j < nrb) {
#pragma unroll
        for (int q = 0; q < GS / 2; ++q) acc ^= wb[i].q[q].x ^ wb[i].q[q].y ^ wb[i].q[q].z ^ wb[i].q[q].w ^ wb[i].d[q];
      }
      issue(j + D, wb[i]);
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// y[i] = sum_{s < S} part[s][i], ascending s.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                             float* __restrict__ y, int64_t n,
                                                             int S) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float t = part[i];
  for (int s = 1; s < S; ++s) t += part[(int64_t)s * n + i];
  y[i] = t;
}

// ---------------------------------------------------------------------------
// host side

int launch_splitk_reduce(const float* part, float* y, int64_t n, int S, hipStream_t st) {
  if (n <= 0) return 0;
  splitk_reduce_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(part, y, n, S);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// rows per unit of the row split (see WgRows)
static int row_unit(int fmt) { return fmt == kFmtPQ2 ? 16 : 4; }
static int64_t row_units(int fmt, int64_t N) { return (N + row_unit(fmt) - 1) / row_unit(fmt); }
// most 16-row blocks a workgroup of `grid` over `units` row units can touch
// (its rows start at most kRB - unit rows into their first block)
static int64_t wg_blocks(int fmt, int64_t units, int64_t grid) {
  const int u = row_unit(fmt);
  const int64_t rows = (units + grid - 1) / grid * u;
  return (kRB - u + rows + kRB - 1) / kRB;
}
static bool few_blocks(int fmt, int64_t units, int64_t grid) {
  static_assert(Pq2Cfg<8>::D == Pq2Cfg<16>::D, "one depth for both prologue shapes");
  return wg_blocks(fmt, units, grid) <= Pq2Cfg<8>::D;
}

GemvPlan plan_gemv(int fmt, int64_t M, int64_t N, int64_t K, int block_len, int split_req) {
  GemvPlan p{};
  p.split = -1;
  const bool pq2 = fmt == kFmtPQ2;
  const int GROUP = pq2 ? 128 : 32;
  const int n = block_len > 1 ? block_len : 1;
  // PQ2_0: half-word lanes unless a rotation block needs a whole wave
  const int epl = pq2 ? (n <= 512 ? 8 : 16) : 0;
  const int GS = pq2 ? (epl == 8 ? Pq2Cfg<8>::GS : Pq2Cfg<16>::GS) : q8_gs((int)M);
  const int MAXW = pq2 ? (epl == 8 ? Pq2Cfg<8>::MAXW : Pq2Cfg<16>::MAXW) : q8_maxw((int)M);
  const int G = (int)(K / GROUP);
  // the PQ2_0 kernels take the slice bounds as two 16-bit halves
  if (pq2 && G >= 65536) return p;
  const int U = n > GROUP ? n / GROUP : 1;
  const int NU = G / U;
  auto waves_for = [&](int S) {
    const int gmax = (NU + S - 1) / S * U;
    return (gmax + GS - 1) / GS;
  };
  auto lds_for = [&](int S) {
    const int nw = waves_for(S);
    return pq2 ? pq2_lds_bytes((int)M, nw, GS)
               : (M <= 4 ? q8_lds_bytes((int)M, nw, GS) : q8b_lds_bytes((int)M, nw, GS));
  };
  auto fits = [&](int S) { return waves_for(S) <= MAXW && lds_for(S) <= kLdsBudget; };
  int S;
  if (split_req > 0) {
    S = split_req;
    if (S > NU || !fits(S)) return p;
  } else {
    S = 1;
    while (S <= NU && !fits(S)) ++S;
    if (S > NU) return p;
  }
  p.split = S;
  p.epl = epl;
  p.gs = GS;
  p.units = U;
  p.nw = waves_for(S);
  p.lds_bytes = lds_for(S);
  // Slices in units of lcm(U, GS) groups start every wave on a multiple of
  // GS, so that its scales are whole aligned runs; taken when that unit still
  // allows S slices and they fit.
  {
    int ua = U;
    while (ua % GS) ua += U;
    const int NA = G % ua == 0 ? G / ua : 0;
    if (ua != U && S <= NA) {
      const int nwa = ((NA + S - 1) / S * ua + GS - 1) / GS;
      const int ldsa = pq2 ? pq2_lds_bytes((int)M, nwa, GS)
                           : (M <= 4 ? q8_lds_bytes((int)M, nwa, GS) : q8b_lds_bytes((int)M, nwa, GS));
      if (nwa <= MAXW && ldsa <= kLdsBudget) {
        p.units = ua;
        p.nw = nwa;
        p.lds_bytes = ldsa;
      }
    }
  }
  const int NUp = G / p.units;
  // row indices are 32-bit in the kernels
  if (N > (int64_t(1) << 31) - 2 * kRB) return p;
  p.total_rb = (int)((N + kRB - 1) / kRB);
  // PQ2_0: every K slice gets the whole grid.  Its waves need at most 168
  // VGPRs, so a compute unit holds two slices' 5-wave workgroups (S = 2) or
  // four 3-wave ones (S = 4), and a split adds waves instead of thinning them
  // (248320 rows: S = 2 64.8 -> 58.4 us, S = 4 99.6 -> 62.7).  Q8_0 keeps one
  // grid in total, which measured faster (17408 rows, M = 4, S = 2: 25.0 against
  // 31.8 us; M = 8: 26.1 against 34.6, whose 256-VGPR waves leave room for one
  // 5-wave workgroup per compute unit).
  const int target = pq2 ? kTargetWGs : (kTargetWGs / S > 0 ? kTargetWGs / S : 1);
  p.grid_x = p.total_rb < target ? p.total_rb : target;
  // a workgroup's rows must fit its buffer resources (see kFarRows)
  const int64_t row_bytes = pq2 ? K / 4 : K;
  const int64_t units = row_units(fmt, N);
  const int64_t wg_rb = wg_blocks(fmt, units, p.grid_x);
  p.few = pq2 && few_blocks(fmt, units, p.grid_x);
  if (wg_rb * kRB * row_bytes > kMaxWgBytes) {
    p.split = -1;
    return p;
  }
  // a wave's scales are whole aligned runs when every slice starts on a
  // multiple of GS groups (waves then start on multiples of GS)
  bool even = true;
  for (int s = 0; s < S && even; ++s) even = part_start(s, NUp / S, NUp % S) * p.units % GS == 0;
  p.dalign = even;
  return p;
}

int64_t gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int block_len,
                             int split_req) {
  GemvPlan p = plan_gemv(fmt, M, N, K, block_len, split_req);
  if (p.split < 1) return -1;
  return p.split > 1 ? (int64_t)p.split * M * N * 4 : 0;
}

template <typename Kernel>
static int launch_kernel(Kernel k, const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  // more than 64 KiB of dynamic LDS needs the attribute
  if (p.lds_bytes > 64 * 1024 &&
      hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) !=
          hipSuccess)
    return -1;
  hipLaunchKernelGGL(k, dim3(p.grid_x, p.split), dim3(p.nw * 64), p.lds_bytes, st, a);
  return 0;
}

// the head of a launch: set 0's planes and rows (several sets read theirs
// from the argument block)
static GemvHead head_of(const GemvArgs& a) {
  GemvHead h;
  h.qs = a.nsets > 1 ? a.set[0].qs : a.qs;
  h.dpl = a.nsets > 1 ? a.set[0].dpl : a.dpl;
  h.x = a.x;
  h.signs = a.signs;
  h.q_base = a.q_base;
  h.q_rem = a.q_rem;
  h.n = (int)a.N;
  h.G = a.G;
  h.u_br = a.u_base | a.u_rem << 16;
  h.unw = a.U;  // | waves << 8, set at launch
  return h;
}

template <typename Kernel>
static int launch_kernel_head(Kernel k, const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  if (p.lds_bytes > 64 * 1024 &&
      hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) !=
          hipSuccess)
    return -1;
  GemvHead h = head_of(a);
  h.unw |= p.nw << 8;
  hipLaunchKernelGGL(k, dim3(p.grid_x, p.split), dim3(p.nw * 64), p.lds_bytes, st, KQ_HEAD_ARGS(h), a);
  return 0;
}

template <int M, int EPL, bool FEW>
static int launch_pq2(const GemvArgs& a, const GemvPlan& p, bool multi, hipStream_t st) {
  return multi ? launch_kernel_head(gemv_pq2_kernel<M, true, EPL, true, FEW>, a, p, st)
         : p.dalign ? launch_kernel_head(gemv_pq2_kernel<M, true, EPL, false, FEW>, a, p, st)
                    : launch_kernel_head(gemv_pq2_kernel<M, false, EPL, false, FEW>, a, p, st);
}

template <int M>
static int launch_m(int fmt, const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  // several sets: one K slice, so every wave starts on a whole scale run
  const bool multi = a.nsets > 1;
  if (multi && !p.dalign) return -2;  // no launch plan for these arguments
  if (fmt == kFmtPQ2) {
    if (p.epl == 8)
      return p.few ? launch_pq2<M, 8, true>(a, p, multi, st) : launch_pq2<M, 8, false>(a, p, multi, st);
    return p.few ? launch_pq2<M, 16, true>(a, p, multi, st) : launch_pq2<M, 16, false>(a, p, multi, st);
  }
  if (p.gs != Q8Cfg<M>::GS) return -2;
  if constexpr (M <= 4)
    return multi ? launch_kernel(gemv_q8_kernel<M, true, true>, a, p, st)
           : p.dalign ? launch_kernel(gemv_q8_kernel<M, true, false>, a, p, st)
                      : launch_kernel(gemv_q8_kernel<M, false, false>, a, p, st);
  else
    return multi ? launch_kernel(gemv_q8_bf16_kernel<M, true, true>, a, p, st)
           : p.dalign ? launch_kernel(gemv_q8_bf16_kernel<M, true, false>, a, p, st)
                      : launch_kernel(gemv_q8_bf16_kernel<M, false, false>, a, p, st);
}

static int launch_args(int fmt, const GemvArgs& a, const GemvPlan& p, int64_t M, hipStream_t st) {
  switch (M) {
    case 1: return launch_m<1>(fmt, a, p, st);
    case 2: return launch_m<2>(fmt, a, p, st);
    case 3: return launch_m<3>(fmt, a, p, st);
    case 4: return launch_m<4>(fmt, a, p, st);
    case 5: return launch_m<5>(fmt, a, p, st);
    case 6: return launch_m<6>(fmt, a, p, st);
    case 7: return launch_m<7>(fmt, a, p, st);
    default: return launch_m<8>(fmt, a, p, st);
  }
}

// fields shared by every weight set: activation, rotation, K geometry
static void common_args(GemvArgs& a, int fmt, const GemvPlan& p, int64_t K, const float* x,
                        int block_len, const int8_t* signs) {
  const PlanarView pv = planar_view(fmt, 1, K, nullptr);
  a.x = x;
  a.signs = signs;
  a.K = K;
  a.row_bytes = (uint32_t)pv.row_bytes;
  a.d_tile_bytes = (uint32_t)pv.d_tile_bytes;
  a.G = (int)(K / (fmt == kFmtPQ2 ? 128 : 32));
  a.U = p.units;
  a.S = p.split;
  a.u_base = (a.G / p.units) / p.split;
  a.u_rem = (a.G / p.units) % p.split;
  int log2n = 0;
  while (block_len > 1 && (1 << log2n) < block_len) ++log2n;
  a.log2n = log2n;
  a.inv_sqrt_n = block_len > 1 ? (float)(1.0 / __builtin_sqrt((double)block_len)) : 1.0f;
  a.nsets = 1;
  a.row_unit = row_unit(fmt);
}

// Workgroups per weight set: the grid of one launch (kTargetWGs) shared in
// proportion to each set's row blocks, at least one and at most one per row
// block each.  Returns the total, or -2 if a set's workgroup slice exceeds
// the buffer-range limit or no single-slice plan fits.
static int multi_split(int fmt, int nsets, const int64_t* N, int64_t K, int64_t M, int block_len,
                       GemvPlan& p, int* wgs) {
  int64_t nmax = 1, total = 0;
  for (int s = 0; s < nsets; ++s) {
    nmax = N[s] > nmax ? N[s] : nmax;
    total += (N[s] + kRB - 1) / kRB;
  }
  p = plan_gemv(fmt, M, nmax, K, block_len, 1);
  if (p.split != 1) return -2;
  const int64_t row_bytes = fmt == kFmtPQ2 ? K / 4 : K;
  int grid = 0;
  bool few = fmt == kFmtPQ2;
  for (int s = 0; s < nsets; ++s) {
    const int64_t rb = (N[s] + kRB - 1) / kRB;
    int64_t w = (kTargetWGs * rb + total / 2) / total;
    w = w < 1 ? 1 : (w > rb ? rb : w);
    const int64_t units = row_units(fmt, N[s]);
    if (wg_blocks(fmt, units, w) * kRB * row_bytes > kMaxWgBytes) return -2;
    few = few && few_blocks(fmt, units, w);
    wgs[s] = (int)w;
    grid += (int)w;
  }
  p.few = few;
  return grid;
}

int check_gemv_multi(int fmt, int nsets, const int64_t* N, int64_t K, int64_t M, int block_len) {
  GemvPlan p;
  int wgs[kMaxSets];
  return multi_split(fmt, nsets, N, K, M, block_len, p, wgs) > 0 ? 0 : -2;
}

int launch_gemv_multi(int fmt, int nsets, const void* const* packed, const int64_t* N, int64_t K,
                      const float* x, int64_t M, int block_len, const int8_t* signs,
                      float* const* y, hipStream_t st) {
  GemvPlan p;
  int wgs[kMaxSets];
  const int grid = multi_split(fmt, nsets, N, K, M, block_len, p, wgs);
  if (grid < 1) return -2;
  GemvArgs a{};
  common_args(a, fmt, p, K, x, block_len, signs);
  a.nsets = nsets;
  int wg0 = 0;
  for (int s = 0; s < kMaxSets; ++s) {
    GemvSet& w = a.set[s];
    if (s < nsets) {
      const PlanarView pv = planar_view(fmt, N[s], K, const_cast<void*>(packed[s]));
      const int units = (int)row_units(fmt, N[s]);
      w.qs = pv.qs;
      w.dpl = pv.d;
      w.out = y[s];
      w.N = N[s];
      w.q_base = units / wgs[s];
      w.q_rem = units % wgs[s];
      w.wg0 = wg0;
      wg0 += wgs[s];
    } else {
      w = a.set[0];
      w.wg0 = 1 << 30;  // never chosen
    }
    w.pad = 0;
  }
  // the single-set fields describe set 0; every workgroup replaces them
  a.qs = a.set[0].qs;
  a.dpl = a.set[0].dpl;
  a.out = a.set[0].out;
  a.N = a.set[0].N;
  a.q_base = a.set[0].q_base;
  a.q_rem = a.set[0].q_rem;
  a.total_rb = 0;
  a.grid_x = grid;
  p.grid_x = grid;
  const int rc = launch_args(fmt, a, p, M, st);
  if (rc) return rc;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemv(int fmt, const void* packed, int64_t N, int64_t K, const float* x, int64_t M,
                int block_len, const int8_t* signs, int split_req, float* y, void* ws,
                hipStream_t st) {
  GemvPlan p = plan_gemv(fmt, M, N, K, block_len, split_req);
  if (p.split < 1) return -2;
  PlanarView pv = planar_view(fmt, N, K, const_cast<void*>(packed));
  GemvArgs a{};
  common_args(a, fmt, p, K, x, block_len, signs);
  a.qs = pv.qs;
  a.dpl = pv.d;
  a.N = N;
  a.total_rb = p.total_rb;
  a.grid_x = p.grid_x;
  a.q_base = (int)(row_units(fmt, N) / p.grid_x);
  a.q_rem = (int)(row_units(fmt, N) % p.grid_x);
  float* part = p.split > 1 ? (float*)ws : nullptr;
  a.out = p.split > 1 ? part : y;
  const int rc = launch_args(fmt, a, p, M, st);
  if (rc) return rc;
  if (hipGetLastError() != hipSuccess) return -1;
  if (p.split > 1) {
    const int64_t n = M * N;
    splitk_reduce_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(part, y, n, p.split);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

int launch_gemv_loads_twin(int fmt, const void* packed, int64_t N, int64_t K, const float* x,
                           int64_t M, int block_len, int split_req, uint32_t* sink, hipStream_t st) {
  GemvPlan p = plan_gemv(fmt, M, N, K, block_len, split_req);
  if (p.split < 1) return -2;
  PlanarView pv = planar_view(fmt, N, K, const_cast<void*>(packed));
  GemvArgs a{};
  common_args(a, fmt, p, K, x, block_len, nullptr);
  a.qs = pv.qs;
  a.dpl = pv.d;
  a.N = N;
  a.out = nullptr;
  a.total_rb = p.total_rb;
  a.grid_x = p.grid_x;
  a.q_base = (int)(row_units(fmt, N) / p.grid_x);
  a.q_rem = (int)(row_units(fmt, N) % p.grid_x);
  const dim3 grid(p.grid_x, p.split), block(p.nw * 64);
  const int m = (int)M;
  if (fmt == kFmtPQ2) {
    constexpr int D = Pq2Cfg<8>::D;
    static_assert(Pq2Cfg<16>::D == D, "one depth for both prologue shapes");
    if (p.epl == 8) {
      if (p.dalign) hipLaunchKernelGGL((gemv_loads_twin_kernel<true, Pq2Cfg<8>::GS, D, true>), grid, block, 0, st, a, m, sink);
      else hipLaunchKernelGGL((gemv_loads_twin_kernel<true, Pq2Cfg<8>::GS, D, false>), grid, block, 0, st, a, m, sink);
    } else {
      if (p.dalign) hipLaunchKernelGGL((gemv_loads_twin_kernel<true, Pq2Cfg<16>::GS, D, true>), grid, block, 0, st, a, m, sink);
      else hipLaunchKernelGGL((gemv_loads_twin_kernel<true, Pq2Cfg<16>::GS, D, false>), grid, block, 0, st, a, m, sink);
    }
  } else {
    constexpr int GS = Q8Cfg<1>::GS;
    static_assert(Q8Cfg<1>::D == 2 && Q8Cfg<8>::D == 2, "two row blocks in flight for 1 and 5..8 rows");
    if (M > 4) {
      constexpr int GS8 = Q8Cfg<8>::GS;
      if (p.dalign) hipLaunchKernelGGL((gemv_loads_twin_kernel<false, GS8, 2, true>), grid, block, 0, st, a, m, sink);
      else hipLaunchKernelGGL((gemv_loads_twin_kernel<false, GS8, 2, false>), grid, block, 0, st, a, m, sink);
    } else if (M == 1) {
      if (p.dalign) hipLaunchKernelGGL((gemv_loads_twin_kernel<false, GS, 2, true>), grid, block, 0, st, a, m, sink);
      else hipLaunchKernelGGL((gemv_loads_twin_kernel<false, GS, 2, false>), grid, block, 0, st, a, m, sink);
    } else {
      static_assert(Q8Cfg<2>::D == 1 && Q8Cfg<4>::D == 1, "one row block in flight for 2..4 rows");
      if (p.dalign) hipLaunchKernelGGL((gemv_loads_twin_kernel<false, GS, 1, true>), grid, block, 0, st, a, m, sink);
      else hipLaunchKernelGGL((gemv_loads_twin_kernel<false, GS, 1, false>), grid, block, 0, st, a, m, sink);
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kq
