// gemm.hip -- prefill GEMM on bf16 MFMA for PQ2_0 and Q8_0 weights.
//
// y[m][n] = sum_k bf16(deq(W)[n][k]) * bf16(x'[m][k]), fp32 accumulation, with
// deq = (q-1)*d for PQ2_0 (Bonsai ternary g128 page, sec. 3.1) and d*q for
// Q8_0 (Kipp pages, "Weight quantization").  Each weight block is dequantized
// once per LDS tile and the tile is reused by every token row of the
// workgroup (the dequantize-once-per-tile prefill scheme of the Kipp
// Benchmarks page, "Quantized projections on the tensor units"; the Bonsai
// page's tiled ternary GEMM and its chunked prefill, sec. 8.3).
//
// gfx950 design
// -------------
// * Block tiles TM (tokens) x TN (weight rows) x 64 (K), 4 or 8 waves in a
//   WGM x WGN arrangement, each wave owning (TM / WGM) x (TN / WGN) outputs as
//   v_mfma_f32_16x16x32_bf16 accumulators.  Three instances:
//     256 x 160, 8 waves 4 x 2 (64 x 80 each, 20 accumulators): prompts; at
//       M = 2048, N = 10240 that is 512 tiles, two per CU, with no tail.  Two
//       waves per SIMD: while one waits on LDS or a barrier the other issues
//       its MFMAs (with 4 waves of 128 x 80 the matrix cores were busy 42.5%
//       of the time, and the kernel ran 204 us against 188);
//     64 x 64 and 16 x 64, waves 1 x 4 (one 16-column slice each): the
//       64- and 16-token chunks of a chunked prefill, where a 256-token tile
//       would spend 3/4 or 15/16 of its matrix-core work on padding rows.
// * Two LDS stages of x' (bf16) and the dequantized weight tile, 128-byte
//   rows with the 16-byte chunks XOR-swizzled by (row / 2) % 8, so that the
//   16-byte operand reads of 16 rows and the row-contiguous writes are both
//   bank-conflict free without padding.  With 72-element padded rows, a
//   quarter of the LDS cycles were bank conflicts (SQ_LDS_BANK_CONFLICT).
// * Software pipeline, one barrier per K-tile.  The MFMAs always run from
//   registers: while the MFMAs of k-step 0 of tile t run, the operands of its
//   k-step 1 are read, tile t + 1 is dequantized and written to the other
//   stage and tile t + 2 is fetched into the staging registers; after the
//   barrier, the MFMAs of k-step 1 overlap the reads of tile t + 1's k-step 0.
//   The stage written in the first half was last read before the previous
//   barrier.
// * Dequantization, eight weights per unit (a 64-wide K-tile row is 8 units):
//   PQ2_0: fp4 conversion of nibble-spread codes gives c exactly, c*d - d is
//   exact in fp32; Q8_0: each int8 converts exactly and q*d is exact in fp32.
//   v_cvt_pk_bf16_f32 rounds pairs to bf16 (nearest even).
// * All global loads go through buffer resources that cover exactly the
//   tile's valid rows, with the whole offset in the range-checked vector
//   offset, so rows past M or N (and K-tiles past the end) read zeros with no
//   branch.
// * Tile order is XCD-aware: the 8 XCDs each take a contiguous eighth of the
//   token tiles and walk every weight tile over it, so the x' rows stay in
//   that XCD's L2 while the weight tiles stream past.
#include <type_traits>
#include <utility>

#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int TK = 64;
constexpr int ROWB = TK * 2;  // bytes per LDS row (no padding)

template <int FMT, int TM_, int TN_, int WGM_, int WGN_, int WPC_ = 1>
struct GemmCfg {
  static constexpr int WPC = WPC_;  // workgroups resident per compute unit
  static constexpr int TM = TM_, TN = TN_, WGM = WGM_, WGN = WGN_;
  static constexpr int NW = WGM * WGN;                 // waves
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static constexpr int NT = 64 * NW;                   // threads
  static constexpr int RPP = NT / 8;                   // LDS rows staged per pass (8 chunks a row)
  static constexpr int WM = TM / WGM, WN = TN / WGN;   // wave tile
  static constexpr int FM = WM / 16, FN = WN / 16;     // MFMA tiles per wave
  static_assert(FM >= 1 && FN >= 1 && FM * 16 == WM && FN * 16 == WN, "whole MFMA tiles");

  static constexpr int AROWS = TM < RPP ? RPP : TM;    // LDS rows of the x' tile (a whole pass)
  static_assert(AROWS % RPP == 0, "whole passes of x' rows");
  static constexpr int ALOADS = AROWS / RPP;           // 16-byte x' chunks per thread
  // 8-weight units per thread; the last pass may cover only the first
  // UNIT_TAIL threads (whole waves)
  static constexpr int UNITS = (TN * TK / 8 + NT - 1) / NT;
  static constexpr int UNIT_TAIL = TN * TK / 8 - (UNITS - 1) * NT;
  static_assert(UNIT_TAIL % 64 == 0 && TN % 16 == 0 && RPP % 16 == 0, "whole waves, 16-row tiles");
  static constexpr int A_BYTES = AROWS * ROWB;
  static constexpr int B_BYTES = TN * ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  // K slices only for the small token tiles (gemm_split); the prompt tile
  // keeps slice 0 as a constant (its loop scheduled slower with a run-time
  // K range: 209 -> 277 us at 2048 x 10240 x 5120)
  static constexpr bool SPLIT = TM < 256;
};

struct GemmArgs {
  const uint16_t* xb;   // x' bf16 [M][K]
  const uint8_t* qs;    // code plane (16-row tiles)
  const uint8_t* dpl;   // scale plane (16-row x 8-block chunks)
  float* y;             // [M][N]
  int64_t M, N, K;
  int64_t d_per_row;    // blocks per row (K / 128 or K / 32)
  int64_t d_tile_bytes; // scale bytes per 16-row tile
  int mt, nt;           // tile counts
  int S;                // K slices: workgroup b takes tile b % (mt nt), slice b / (mt nt)
  int kt_per;           // K-tiles per slice (even for PQ2_0)
  float* part;          // S > 1: fp32 partials [S][M][N]
};

// 8 PQ2_0 codes (16 bits of a word in the block's own order, code j at bits
// 2j, after pq2_load_word) -> 8 bf16 values (q-1)*d, as 4 dwords in element
// order
__device__ __forceinline__ uint4 dequant8_pq2(uint32_t h, float d) {
  const uint32_t e = h & 0x3333u;         // codes 0, 2, 4, 6 in nibbles 0..3
  const uint32_t o = (h >> 2) & 0x3333u;  // codes 1, 3, 5, 7
  const f32x2 e0 = codes2<0>(e), e1 = codes2<1>(e), o0 = codes2<0>(o), o1 = codes2<1>(o);
  return make_uint4(pack_bf16x2(fmaf(e0.x, d, -d), fmaf(o0.x, d, -d)),
                    pack_bf16x2(fmaf(e0.y, d, -d), fmaf(o0.y, d, -d)),
                    pack_bf16x2(fmaf(e1.x, d, -d), fmaf(o1.x, d, -d)),
                    pack_bf16x2(fmaf(e1.y, d, -d), fmaf(o1.y, d, -d)));
}
// 8 Q8_0 codes (int8, element j in byte j of the pair) -> 8 bf16 values q*d
__device__ __forceinline__ uint4 dequant8_q8(uint2 w, float d) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = (float)(int8_t)(w.x >> (8 * j)) * d;
    v[4 + j] = (float)(int8_t)(w.y >> (8 * j)) * d;
  }
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// buffer loads with the whole offset per lane (range-checked)
__device__ __forceinline__ uint4 load16(BufRsrc r, uint32_t off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load8(BufRsrc r, uint32_t off) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load4(BufRsrc r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t load2(BufRsrc r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

template <typename Cfg, int FMT>
__global__ __launch_bounds__(Cfg::NT, Cfg::WPC) void gemm_kernel(GemmArgs a) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN, WM = Cfg::WM, WN = Cfg::WN, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int ALOADS = Cfg::ALOADS, UNITS = Cfg::UNITS, RPP = Cfg::RPP;
  constexpr int A_BYTES = Cfg::A_BYTES, STAGE_BYTES = Cfg::STAGE_BYTES;
  constexpr bool PQ2 = FMT == kFmtPQ2;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;

  // ---- K slice and XCD-aware tile mapping
  const int tiles = a.mt * a.nt;
  const int slice = Cfg::SPLIT ? (int)blockIdx.x / tiles : 0;
  const int bid = (int)blockIdx.x - slice * tiles;
  int m_tile, n_tile;
  if ((a.mt & 7) == 0) {
    // XCD x takes an eighth of the token tiles and walks every weight tile
    // over them: its x' rows stay in its L2 while the weight tiles stream past
    const int xcd = bid & 7, local = bid >> 3;
    m_tile = xcd * (a.mt >> 3) + local / a.nt;
    n_tile = local % a.nt;
  } else if ((a.nt & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3;
    const int npx = a.nt >> 3;
    n_tile = xcd * npx + local % npx;
    m_tile = local / npx;
  } else {
    n_tile = bid % a.nt;
    m_tile = bid / a.nt;
  }
  const int64_t m0 = (int64_t)m_tile * TM, n0 = (int64_t)n_tile * TN;

  // ---- global load geometry.  Thread t stages x' chunk t % 8 (8 bf16) of
  // rows t / 8 + RPP i, and weight units (rows t / 8 + RPP i, chunk t % 8),
  // RPP = threads / 8 rows a pass.
  // K order inside a tile: PQ2_0 interleaves the two K-tiles of a 128-block in
  // runs of 8 (chunk c of K-tile 2b + h holds elements 16 c + 8 h .. + 7 of
  // block b), so that one 4-byte word per unit brings a thread's codes for
  // both K-tiles; Q8_0 keeps the natural order (chunk c of K-tile t holds
  // elements 64 t + 8 c .. + 7, bytes 8 (c % 4) .. + 7 of block 2 t + c / 4).
  // The product is a sum over K, so any order shared by both operands gives it.
  const int arow = tid >> 3, achunk = tid & 7;
  const int64_t G = a.d_per_row;
  const int64_t arows = a.M - m0 < TM ? a.M - m0 : TM;
  const int64_t brows = a.N - n0 < TN ? a.N - n0 : TN;
  const BufRsrc ra_rs = make_rsrc(a.xb + m0 * a.K, (uint32_t)(arows * a.K * 2));
  const BufRsrc rq_rs = make_rsrc(a.qs + (n0 >> 4) * G * 512, (uint32_t)((brows + 15) / 16 * G * 512));
  const BufRsrc rd_rs = make_rsrc(a.dpl + (n0 >> 4) * a.d_tile_bytes, (uint32_t)((brows + 15) / 16 * a.d_tile_bytes));
  const uint32_t a_off = (uint32_t)(arow * a.K + achunk * (PQ2 ? 16 : 8)) * 2u;
  const uint32_t rowstep = (uint32_t)(RPP * a.K * 2);
  // unit i: weight row RPP i + t / 8 = 16-row tile (t / 128 + RPP / 16 i), row (t / 8) % 16
  const uint32_t q_off = PQ2 ? (uint32_t)((tid >> 7) * G * 512 + ((tid >> 3) & 15) * 32 + achunk * 4)
                             : (uint32_t)((tid >> 7) * G * 512 + ((tid >> 3) & 15) * 32 + (achunk & 3) * 8 +
                                          (achunk >> 2) * 512);
  const uint32_t q_step = (uint32_t)(RPP / 16 * G * 512);  // a pass of 16-row tiles
  const uint32_t d_off = (uint32_t)((tid >> 7) * a.d_tile_bytes + ((tid >> 3) & 15) * 16);
  const uint32_t d_step = (uint32_t)(RPP / 16 * a.d_tile_bytes);
  // K-tiles: PQ2_0 has an even number (K is a multiple of 128); Q8_0 may end
  // in half a tile (K a multiple of 32), whose chunks past K load nothing.
  // This workgroup's slice: K-tiles [kt0, kt1) (kt0 even for PQ2_0).
  const int KTall = (int)((a.K + TK - 1) / TK);
  const int kt0 = Cfg::SPLIT ? slice * a.kt_per : 0;
  const int kt1 = Cfg::SPLIT && kt0 + a.kt_per < KTall ? kt0 + a.kt_per : KTall;
  const int KT = kt1 - kt0;

  // LDS byte offset of this thread's 16-byte chunk in rows arow + RPP i:
  // row * 128 + (chunk ^ (row / 2) % 8) * 16, and (row / 2) % 8 = (t / 16) % 8
  const uint32_t w_lds = (uint32_t)(arow * ROWB + ((achunk ^ ((tid >> 4) & 7)) << 4));

  // staging registers: the tile written to LDS at the start of iteration t
  // was fetched at the start of iteration t - 1 (PQ2_0: a block's words and
  // scales are fetched with its even K-tile and serve both)
  uint4 ra[ALOADS];
  uint32_t rq[PQ2 ? UNITS : 1];
  uint2 rq8[PQ2 ? 1 : UNITS];
  uint32_t rdd[UNITS];
  // the staging in pieces: x' chunk i and weight unit i of a K-tile
  auto gload_a = [&](int t, int i) __attribute__((always_inline)) {
    // absolute K-tile; the prefetches of the last two iterations load nothing
    const int kt = kt0 + t;
    const bool in_k = PQ2 ? kt < kt1 : kt < kt1 && (int64_t)kt * TK + 8 * achunk < a.K;
    const uint32_t ak = PQ2 ? a_off + (uint32_t)(((kt >> 1) * 128 + (kt & 1) * 8) * 2)
                            : a_off + (uint32_t)(kt * TK * 2);
    // rows past TM (the 16-token tile stages 32 LDS rows) load nothing
    const bool in_m = RPP * i + arow < TM;
    ra[i] = load16(ra_rs, in_k && in_m ? ak + i * rowstep : kOutOfRange);
  };
  // the last pass of weight units covers the first UNIT_TAIL threads
  auto unit_ok = [&](int i) __attribute__((always_inline)) {
    return Cfg::UNIT_TAIL == Cfg::NT || i < UNITS - 1 || tid < Cfg::UNIT_TAIL;
  };
  auto gload_b = [&](int t, int i) __attribute__((always_inline)) {
    const int kt = kt0 + t;
    const bool in_k = (PQ2 ? kt < kt1 : kt < kt1 && (int64_t)kt * TK + 8 * achunk < a.K) && unit_ok(i);
    if constexpr (PQ2) {
      if ((kt & 1) == 0) {
        const uint32_t kb = (uint32_t)kt >> 1;
        const uint32_t qk = q_off + kb * 512;
        const uint32_t dk = d_off + (kb >> 3) * 256 + (kb & 7) * 2;
        rq[i] = load4(rq_rs, in_k ? qk + i * q_step : kOutOfRange);
        rdd[i] = load2(rd_rs, in_k ? dk + i * d_step : kOutOfRange);
      }
    } else {
      // the unit's 32-block: 2 kt + chunk / 4
      const uint32_t b = 2u * (uint32_t)kt + ((uint32_t)achunk >> 2);
      const uint32_t qk = q_off + (uint32_t)kt * 1024u;
      const uint32_t dk = d_off + (b >> 3) * 256 + (b & 7) * 2;
      rq8[i] = load8(rq_rs, in_k ? qk + i * q_step : kOutOfRange);
      rdd[i] = load2(rd_rs, in_k ? dk + i * d_step : kOutOfRange);
    }
  };
  auto gload = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < ALOADS; ++i) gload_a(t, i);
#pragma unroll
    for (int i = 0; i < UNITS; ++i) gload_b(t, i);
  };
  auto sstore_a = [&](int stage, int i) __attribute__((always_inline)) {
    *reinterpret_cast<uint4*>(smem + stage * STAGE_BYTES + w_lds + i * RPP * ROWB) = ra[i];
  };
  auto sstore_b = [&](int stage, int kt, int i) __attribute__((always_inline)) {
    if (!unit_ok(i)) return;
    const float d = f16_bits_to_f32(rdd[i]);
    uint4 v;
    if constexpr (PQ2) v = dequant8_pq2(pq2_load_word(rq[i]) >> (16 * (kt & 1)), d);
    else v = dequant8_q8(rq8[i], d);
    *reinterpret_cast<uint4*>(smem + stage * STAGE_BYTES + A_BYTES + w_lds + i * RPP * ROWB) = v;
  };
  auto sstore = [&](int stage, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < ALOADS; ++i) sstore_a(stage, i);
#pragma unroll
    for (int i = 0; i < UNITS; ++i) sstore_b(stage, kt, i);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // operand rows: lane (r, kq) reads 8 bf16 at k = 32 ks + 8 kq of row r of a
  // 16-row tile; swizzled chunk (4 ks + kq) ^ (r / 2) % 8 (rows of a tile
  // start at multiples of 16, so (row / 2) % 8 = (r / 2) % 8)
  const int fr = lane & 15, kq = lane >> 4;
  const uint32_t sw = (uint32_t)((kq ^ (fr >> 1)) & 7) << 4;
  // k-step 1 flips chunk bit 2 (byte 64); row and tile offsets leave it clear
  const uint32_t a_rd0 = (uint32_t)((wm * WM + fr) * ROWB) + sw;
  const uint32_t b_rd0 = (uint32_t)(A_BYTES + (wn * WN + fr) * ROWB) + sw;
  const uint32_t a_rd1 = a_rd0 ^ 64u, b_rd1 = b_rd0 ^ 64u;
  // one set of A operands, refilled row tile by row tile as the MFMAs release
  // them; two sets of B operands (all are used by every row tile)
  bf16x8 fa[FM], fb[2][FN];
  auto lda = [&](int stage, int ks, int i) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(smem + stage * STAGE_BYTES + (ks ? a_rd1 : a_rd0) + i * 16 * ROWB);
  };
  auto ldb = [&](int stage, int ks, int j) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(smem + stage * STAGE_BYTES + (ks ? b_rd1 : b_rd0) + j * 16 * ROWB);
  };
  // the MFMAs of one k-step with B set `cur`, reading the operands of the next
  // k-step (stage `ns`, k-step `nks`) into A and B set `cur ^ 1`
  auto mma = [&](int cur, int ns, int nks) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[cur][j], acc[i][j], 0, 0, 0);
      fa[i] = lda(ns, nks, i);
      if (i < FN) fb[cur ^ 1][i] = ldb(ns, nks, i);
      // B operands past the last row tile are read with the first ones
      if (FM + i < FN) fb[cur ^ 1][FM + i] = ldb(ns, nks, FM + i);
    }
    static_assert(FN <= 2 * FM, "every B operand read in a row tile");
  };
  // prologue: tiles 0 and 1 to stages 0 and 1, tiles 2 and 3 in flight,
  // the first k-step's operands in registers
  gload(0);
  sstore(0, 0);
  gload(1);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[i] = lda(0, 0, i);
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[0][j] = ldb(0, 0, j);

  // iteration t: stage t % 2 holds tile t.  First half: k-step 0 of tile t
  // from registers while its k-step 1 is read, tile t + 1 (fetched during the
  // last iteration) is written to the other stage and tile t + 2 is fetched.
  // Second half, after the barrier: k-step 1 while the next tile's k-step 0 is
  // read.  The other stage was last read before the previous barrier, so one
  // barrier per tile suffices.
  // k-step 0 of the 256 x 160 tile with the staging cut into its rows: after
  // the MFMAs of row tile i and the reads of its next operands, x' chunk i and
  // weight unit i of tile t + 1 go to LDS and those of tile t + 2 are fetched
  auto half0_staged = [&](int st, int t) __attribute__((always_inline)) {
    static_for<FM>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[0][j], acc[i][j], 0, 0, 0);
      fa[i] = lda(st, 1, i);
      if constexpr (i < FN) fb[1][i] = ldb(st, 1, i);
      if constexpr (FM + i < FN) fb[1][FM + i] = ldb(st, 1, FM + i);
      if constexpr (i < ALOADS) {
        sstore_a(st ^ 1, i);
        gload_a(t + 2, i);
      }
      if constexpr (i < UNITS) {
        sstore_b(st ^ 1, t + 1, i);
        gload_b(t + 2, i);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto iter = [&](int t, auto STAGE) __attribute__((always_inline)) {
    constexpr int st = decltype(STAGE)::value;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TM == 256) {
      static_assert(FM >= ALOADS && FM >= UNITS, "a staging piece per row tile");
      half0_staged(st, t);
    } else {
      sstore(st ^ 1, t + 1);
      gload(t + 2);
      mma(0, st, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    mma(1, st ^ 1, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // the last tiles are peeled off the loop: with them inside, the compiler
  // moved the accumulators between register files every iteration
  int t = 0;
  for (; t + 2 < KT; t += 2) {
    iter(t, std::integral_constant<int, 0>{});
    iter(t + 1, std::integral_constant<int, 1>{});
  }
  if (t + 1 < KT) {
    iter(t, std::integral_constant<int, 0>{});
    iter(t + 1, std::integral_constant<int, 1>{});
  } else {
    iter(t, std::integral_constant<int, 0>{});  // Q8_0 with an odd number of K-tiles
  }

  // ---- epilogue: lane (j, q), register r -> row 4q + r, column j of a tile
  float* out = Cfg::SPLIT && a.S > 1 ? a.part + (int64_t)slice * a.M * a.N : a.y;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * WN + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + r;
        if (row < a.M && col < a.N) out[row * a.N + col] = acc[i][j][r];
      }
    }
  }
}

// Token-tile instances: the 256 x 160 prompt tile, and 64- / 16-token tiles
// of 64 weight rows for short chunks.
template <int FMT> using CfgBig = GemmCfg<FMT, 256, 160, 4, 2>;
template <int FMT> using Cfg64 = GemmCfg<FMT, 64, 64, 1, 4>;
template <int FMT> using Cfg16 = GemmCfg<FMT, 16, 64, 1, 4>;

// token tile for M tokens: 16 up to 16, 64 up to 96, else 256
static int gemm_tile_m(int64_t M) { return M <= 16 ? 16 : (M <= 96 ? 64 : 256); }
static int gemm_tile_n(int tm) { return tm == 256 ? 160 : 64; }

// K slices of the small token tiles.  A 16- or 64-token tile has little work
// per K-tile, so its loop waits on memory each K-tile; the N / 64 tiles of one
// chunk leave most compute units idle.  Splitting K until there are up to
// four workgroups per compute unit (1024: one round, as four 64-token
// workgroups fit a compute unit), in slices of whole K-tile pairs for PQ2_0,
// gives each workgroup about a sixth of the loop; the fp32 partials are
// added in slice order by a second kernel (deterministic).
struct GemmSplit {
  int S, kt_per;
};
static GemmSplit gemm_split(int fmt, int64_t M, int64_t N, int64_t K) {
  const int tm = gemm_tile_m(M), tn = gemm_tile_n(tm);
  const int64_t KT = (K + TK - 1) / TK;
  const int64_t tiles = ((M + tm - 1) / tm) * ((N + tn - 1) / tn);
  if (tm == 256 || tiles >= 1024) return {1, (int)KT};
  const int unit = fmt == kFmtPQ2 ? 2 : 1;
  const int64_t units = (KT + unit - 1) / unit;
  int64_t S = 1024 / tiles;
  S = S < units ? S : units;
  S = S < 16 ? S : 16;
  const int64_t kt_per = (units + S - 1) / S * unit;
  return {(int)((KT + kt_per - 1) / kt_per), (int)kt_per};
}

// 32-bit buffer ranges and offsets: a 256-row x' tile spans 512 K bytes,
// which must stay below the out-of-range offset (kOutOfRange, about 2^31);
// the tile grid must fit an int.
bool gemm_shape_supported(int64_t M, int64_t N, int64_t K) {
  if (K > kGemmMaxK) return false;
  const int tm = gemm_tile_m(M), tn = gemm_tile_n(tm);
  const int64_t mt = (M + tm - 1) / tm, nt = (N + tn - 1) / tn;
  return mt * nt <= 0x7FFFFFFF;
}

int gemm_split_count(int fmt, int64_t M, int64_t N, int64_t K) { return gemm_split(fmt, M, N, K).S; }

// x' (bf16 [M][K], 256-byte aligned), then the split partials (fp32 [S][M][N])
static int64_t gemm_xb_bytes(int64_t M, int64_t K) { return (M * K * 2 + 255) / 256 * 256; }
int64_t gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int block_len, int x_bf16,
                             const void* signs_hint) {
  (void)block_len; (void)x_bf16; (void)signs_hint;
  const GemmSplit sp = gemm_split(fmt, M, N, K);
  return gemm_xb_bytes(M, K) + (sp.S > 1 ? (int64_t)sp.S * M * N * 4 : 0);
}

template <typename Cfg, int FMT>
static int launch_tile(const GemmArgs& base, hipStream_t st) {
  GemmArgs a = base;
  a.mt = (int)((a.M + Cfg::TM - 1) / Cfg::TM);
  a.nt = (int)((a.N + Cfg::TN - 1) / Cfg::TN);
  // more than 64 KiB of dynamic LDS needs the attribute; set once per
  // instance (thread-safe static initialisation)
  static const bool attr_ok =
      Cfg::LDS_BYTES <= 64 * 1024 ||
      hipFuncSetAttribute((const void*)gemm_kernel<Cfg, FMT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          Cfg::LDS_BYTES) == hipSuccess;
  if (!attr_ok) return -1;
  gemm_kernel<Cfg, FMT><<<a.mt * a.nt * a.S, Cfg::NT, Cfg::LDS_BYTES, st>>>(a);
  if (hipGetLastError() != hipSuccess) return -1;
  return a.S > 1 ? launch_splitk_reduce(a.part, a.y, a.M * a.N, a.S, st) : 0;
}

template <int FMT>
static int launch_fmt(const GemmArgs& a, hipStream_t st) {
  switch (gemm_tile_m(a.M)) {
    case 16: return launch_tile<Cfg16<FMT>, FMT>(a, st);
    case 64: return launch_tile<Cfg64<FMT>, FMT>(a, st);
    default: return launch_tile<CfgBig<FMT>, FMT>(a, st);
  }
}

int launch_gemm(int fmt, const void* packed, int64_t N, int64_t K, const void* x, int x_bf16,
                int64_t M, int block_len, const int8_t* signs, float* y, void* ws, hipStream_t st) {
  const uint16_t* xb = (const uint16_t*)x;
  if (block_len > 0 || signs || !x_bf16) {
    if (launch_hadamard(x, x_bf16, ws, 1, M, K, block_len > 0 ? block_len : 1, signs, st)) return -1;
    xb = (const uint16_t*)ws;
  }
  PlanarView pv = planar_view(fmt, N, K, const_cast<void*>(packed));
  GemmArgs a;
  a.xb = xb;
  a.qs = pv.qs;
  a.dpl = pv.d;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  a.d_per_row = pv.d_per_row;
  a.d_tile_bytes = pv.d_tile_bytes;
  a.mt = a.nt = 0;
  const GemmSplit sp = gemm_split(fmt, M, N, K);
  a.S = sp.S;
  a.kt_per = sp.kt_per;
  a.part = sp.S > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + gemm_xb_bytes(M, K)) : nullptr;
  return fmt == kFmtPQ2 ? launch_fmt<kFmtPQ2>(a, st) : launch_fmt<kFmtQ8>(a, st);
}

}  // namespace kq
