// gemm.hip -- PQ2_0 prefill GEMM on bf16 MFMA.
//
// y[m][n] = sum_k bf16((q-1)*d)[n][k] * bf16(x'[m][k]), fp32 accumulation.
// Each weight block is dequantized once per LDS tile and the tile is reused
// by every token row of the workgroup (the dequantize-once-per-tile prefill
// scheme of the Kipp Benchmarks page, "Quantized projections on the tensor
// units"; the Bonsai page's tiled ternary GEMM, sec. 8.3, 8.5).
//
// gfx950 design
// -------------
// * Block tile 256 (tokens) x 160 (weight rows) x 64 (K), 4 waves in a 2 x 2
//   arrangement; each wave owns 128 x 80 outputs = 8 x 5 accumulators of
//   v_mfma_f32_16x16x32_bf16 (160 fp32 registers).  At M = 2048, N = 10240
//   that is 512 tiles, two per CU, with no tail imbalance.
// * Two LDS stages of x' (bf16) and the dequantized weight tile, 128-byte
//   rows with the 16-byte chunks XOR-swizzled by (row / 2) % 8, so that the
//   16-byte operand reads of 16 rows and the row-contiguous writes are both
//   bank-conflict free without padding (2 x 52 KiB).  With the 72-element
//   padded rows used before, a quarter of the LDS cycles were bank
//   conflicts (SQ_LDS_BANK_CONFLICT).
// * Software pipeline, one barrier per K-tile.  The MFMAs always run from
//   registers: while the 40 MFMAs of k-step 0 of tile t run, the operands of
//   its k-step 1 are read, tile t + 1 is dequantized and written to the
//   other stage and tile t + 2 is fetched into the staging registers; after
//   the barrier, the 40 MFMAs of k-step 1 overlap the reads of tile t + 1's
//   k-step 0.  The stage written in the first half was last read before the
//   previous barrier.
// * Dequantization: the 160 x 64 codes of a tile are 1280 units of 8 codes,
//   five per thread: fp4 conversion of the nibble-spread codes gives c
//   exactly, c*d - d is exact in fp32, and v_cvt_pk_bf16_f32 rounds pairs to
//   bf16 (nearest even) -- the same value as (q-1) * bf16(d).
// * Tile order is XCD-aware: the 8 XCDs each take a contiguous eighth of the
//   token tiles and walk every weight tile over it, so the x' rows stay in
//   that XCD's L2 while the (ten times smaller) weight tiles stream past.
#include <type_traits>

#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int TM = 256, TN = 160, TK = 64;
constexpr int ROWB = TK * 2;                        // bytes per LDS row (no padding)
constexpr int A_BYTES = TM * ROWB;                  // 32 KiB
constexpr int B_BYTES = TN * ROWB;                  // 20 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;      // 52 KiB
constexpr int NSTAGE = 2;
constexpr int GEMM_LDS_BYTES = NSTAGE * STAGE_BYTES;
constexpr int WM = TM / 2, WN = TN / 2;             // wave tile 128 x 80
constexpr int FM = WM / 16, FN = WN / 16;           // 8 x 5 MFMA tiles per wave
constexpr int UNITS = TN * TK / 8 / 256;            // 8-code units per thread per tile (5)
static_assert(TN * TK / 8 == UNITS * 256, "units must divide evenly");

struct GemmArgs {
  const uint16_t* xb;   // x' bf16 [M][K]
  const uint8_t* qs;    // code plane (16-row tiles)
  const uint8_t* dpl;   // scale plane (16-row x 8-block chunks)
  float* y;             // [M][N]
  int64_t M, N, K;
  int64_t d_per_row;    // blocks per row (K / 128)
  int64_t d_tile_bytes; // scale bytes per 16-row tile
  int mt, nt;           // tile counts
};

// 8 codes (16 bits, code j at bits 2j) -> 8 bf16 values (q-1)*d, as 4 dwords
// in element order
__device__ __forceinline__ uint4 dequant8_bf16(uint32_t h, float d) {
  const uint32_t e = h & 0x3333u;         // codes 0, 2, 4, 6 in nibbles 0..3
  const uint32_t o = (h >> 2) & 0x3333u;  // codes 1, 3, 5, 7
  const f32x2 e0 = codes2<0>(e), e1 = codes2<1>(e), o0 = codes2<0>(o), o1 = codes2<1>(o);
  return make_uint4(pack_bf16x2(fmaf(e0.x, d, -d), fmaf(o0.x, d, -d)),
                    pack_bf16x2(fmaf(e0.y, d, -d), fmaf(o0.y, d, -d)),
                    pack_bf16x2(fmaf(e1.x, d, -d), fmaf(o1.x, d, -d)),
                    pack_bf16x2(fmaf(e1.y, d, -d), fmaf(o1.y, d, -d)));
}

// buffer loads with a per-thread offset and a uniform (scalar) one
__device__ __forceinline__ uint4 load16_s(BufRsrc r, uint32_t voff, uint32_t soff) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load4_s(BufRsrc r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t load2_s(BufRsrc r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

__global__ __launch_bounds__(256, 1) void gemm_pq2_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- XCD-aware tile mapping
  const int bid = blockIdx.x;
  int m_tile, n_tile;
  if ((a.mt & 7) == 0) {
    // XCD x takes an eighth of the token tiles and walks every weight tile
    // over them: its x' rows (2.6 MB per token tile at K = 5120) stay in its
    // L2 while the weight tiles, a tenth of the size, stream past
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

  // ---- global load geometry.  K order inside a tile: the two K-tiles of a
  // 128-element block interleave in runs of 8, so chunk c (8 elements) of
  // K-tile 2b + h holds elements 16 c + 8 h .. +7 of block b.  The product
  // is a sum over K, so any order shared by both operands gives it; this one
  // puts a thread's codes for both K-tiles of a block in one 4-byte word.
  // x' tile: load i of thread t covers row 32 i + t / 8, chunk t % 8.
  // Weights: unit i of thread t is weight row 32 i + t / 8, chunk t % 8: 16
  // bits of a 4-byte word loaded once per block (the low half for the even
  // K-tile), with the block's scale.
  // All go through buffer resources that cover exactly the block's valid
  // rows (the code and scale resources: its valid 16-row tiles, whose rows
  // past N hold zero codes and zero scales), with the whole offset in the
  // range-checked vector offset, so rows past M or N read zeros with no
  // branch: code 0 with scale 0 dequantizes to 0.
  const int arow = tid >> 3, achunk = tid & 7;
  const int64_t G = a.d_per_row;
  const int64_t arows = a.M - m0 < TM ? a.M - m0 : TM;
  const int64_t brows = a.N - n0 < TN ? a.N - n0 : TN;
  const BufRsrc ra_rs = make_rsrc(a.xb + m0 * a.K, (uint32_t)(arows * a.K * 2));
  const BufRsrc rq_rs = make_rsrc(a.qs + (n0 >> 4) * G * 512, (uint32_t)((brows + 15) / 16 * G * 512));
  const BufRsrc rd_rs = make_rsrc(a.dpl + (n0 >> 4) * a.d_tile_bytes, (uint32_t)((brows + 15) / 16 * a.d_tile_bytes));
  const uint32_t a_off = (uint32_t)(arow * a.K + achunk * 16) * 2u;
  // unit i: row 32 i + t / 8 = 16-row tile (t / 128 + 2 i), row (t / 8) % 16
  const uint32_t q_off = (uint32_t)((tid >> 7) * G * 512 + ((tid >> 3) & 15) * 32 + achunk * 4);
  const uint32_t q_step = (uint32_t)(2 * G * 512);  // two 16-row tiles
  const uint32_t d_off = (uint32_t)((tid >> 7) * a.d_tile_bytes + ((tid >> 3) & 15) * 16);
  const uint32_t d_step = (uint32_t)(2 * a.d_tile_bytes);

  // LDS byte offset of this thread's 16-byte chunk in rows arow + 32 i (A)
  // and in weight rows arow + 32 i (B): row * 128 + (chunk ^ (row / 2) % 8) * 16,
  // and (row / 2) % 8 = (t / 16) % 8 for every i
  const uint32_t w_lds = (uint32_t)(arow * ROWB + ((achunk ^ ((tid >> 4) & 7)) << 4));

  // staging registers: the tile written to LDS at the start of iteration t
  // was fetched at the start of iteration t - 1; the weight words and scales
  // of a block are fetched with its even K-tile and serve both
  const int KT = (int)(a.K / TK);  // even: K is a multiple of 128
  uint4 ra[8];
  uint32_t rq[UNITS];
  uint32_t rdd[UNITS];
  // Every offset goes into the per-lane (vector) offset: the hardware range
  // check of a raw buffer load covers the vector offset only, not the scalar
  // one.  K-tiles past the end (the prefetches of the last two iterations)
  // load at kOutOfRange.
  auto gload = [&](int kt, bool with_b) {
    const bool in_k = kt < KT;
    const uint32_t kb = (uint32_t)kt >> 1, h = (uint32_t)kt & 1u;
    const uint32_t rowstep = (uint32_t)(32 * a.K * 2);
    const uint32_t ak = a_off + (kb * 128 + h * 8) * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = load16_s(ra_rs, in_k ? ak + i * rowstep : kOutOfRange, 0);
    if (with_b) {
      const uint32_t qk = q_off + kb * 512;
      const uint32_t dk = d_off + (kb >> 3) * 256 + (kb & 7) * 2;
#pragma unroll
      for (int i = 0; i < UNITS; ++i) {
        rq[i] = load4_s(rq_rs, in_k ? qk + i * q_step : kOutOfRange, 0);
        rdd[i] = load2_s(rd_rs, in_k ? dk + i * d_step : kOutOfRange, 0);
      }
    }
  };
  auto sstore = [&](int stage, int h) {
    uint8_t* S = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(S + w_lds + i * 32 * ROWB) = ra[i];
#pragma unroll
    for (int i = 0; i < UNITS; ++i)
      *reinterpret_cast<uint4*>(S + A_BYTES + w_lds + i * 32 * ROWB) =
          dequant8_bf16(rq[i] >> (16 * h), f16_bits_to_f32(rdd[i]));
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
  // them; two sets of B operands (all five are used by every row tile)
  bf16x8 fa[FM], fb[2][FN];
  auto lda = [&](int stage, int ks, int i) {
    return *reinterpret_cast<const bf16x8*>(smem + stage * STAGE_BYTES + (ks ? a_rd1 : a_rd0) + i * 16 * ROWB);
  };
  auto ldb = [&](int stage, int ks, int j) {
    return *reinterpret_cast<const bf16x8*>(smem + stage * STAGE_BYTES + (ks ? b_rd1 : b_rd0) + j * 16 * ROWB);
  };
  // the 40 MFMAs of one k-step with B set `cur`, reading the operands of the
  // next k-step (stage `ns`, k-step `nks`) into A and B set `cur ^ 1`
  auto mma = [&](int cur, int ns, int nks) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[cur][j], acc[i][j], 0, 0, 0);
      fa[i] = lda(ns, nks, i);
      if (i < FN) fb[cur ^ 1][i] = ldb(ns, nks, i);
    }
  };

  // prologue: tiles 0 and 1 to stages 0 and 1, tiles 2 and 3 in flight,
  // the first k-step's operands in registers
  gload(0, true);
  sstore(0, 0);
  gload(1, false);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[i] = lda(0, 0, i);
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[0][j] = ldb(0, 0, j);

  // iteration t: stage t % 2 holds tile t.  First half: k-step 0 of tile t
  // from registers while its k-step 1 is read, tile t + 1 (fetched during
  // the last iteration) is written to the other stage and tile t + 2 is
  // fetched.  Second half, after the barrier: k-step 1 while the next tile's
  // k-step 0 is read.  The other stage was last read before the previous
  // barrier, so one barrier per tile suffices.
  auto iter = [&](int t, auto STAGE) {
    constexpr int st = decltype(STAGE)::value;
    __builtin_amdgcn_sched_barrier(0);
    sstore(st ^ 1, st ^ 1);
    gload(t + 2, st == 0);
    mma(0, st, 1);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (j == 1 || j == 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      if (i < FN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    mma(1, st ^ 1, 0);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < FN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // the last two tiles are peeled off the loop: with them inside, the
  // compiler moved the accumulators between register files every iteration
  int t = 0;
  for (; t + 2 < KT; t += 2) {
    iter(t, std::integral_constant<int, 0>{});
    iter(t + 1, std::integral_constant<int, 1>{});
  }
  iter(t, std::integral_constant<int, 0>{});
  iter(t + 1, std::integral_constant<int, 1>{});

  // ---- epilogue: lane (j, q), register r -> row 4q + r, column j of a tile
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * WN + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + r;
        if (row < a.M && col < a.N) a.y[row * a.N + col] = acc[i][j][r];
      }
    }
  }
}

// 32-bit buffer ranges and offsets: a 256-row x' tile spans 512 K bytes,
// which must stay below the out-of-range offset (kOutOfRange, about 2^31);
// the tile grid must fit an int.
bool gemm_shape_supported(int64_t M, int64_t N, int64_t K) {
  if (K > kGemmMaxK) return false;
  const int64_t mt = (M + TM - 1) / TM, nt = (N + TN - 1) / TN;
  return mt * nt <= 0x7FFFFFFF;
}

int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int block_len, int x_bf16,
                             const void* signs_hint) {
  (void)N; (void)block_len; (void)x_bf16; (void)signs_hint;
  return (M * K * 2 + 255) / 256 * 256;
}

int launch_gemm(const void* packed, int64_t N, int64_t K, const void* x, int x_bf16, int64_t M,
                int block_len, const int8_t* signs, float* y, void* ws, hipStream_t st) {
  const uint16_t* xb = (const uint16_t*)x;
  if (block_len > 0 || signs || !x_bf16) {
    if (launch_hadamard(x, x_bf16, ws, 1, M, K, block_len > 0 ? block_len : 1, signs, st)) return -1;
    xb = (const uint16_t*)ws;
  }
  PlanarView pv = planar_view(kFmtPQ2, N, K, const_cast<void*>(packed));
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
  a.mt = (int)((M + TM - 1) / TM);
  a.nt = (int)((N + TN - 1) / TN);
  // the kernel needs more than 64 KiB of dynamic LDS; set once (thread-safe
  // static initialisation)
  static const bool attr_ok =
      hipFuncSetAttribute((const void*)gemm_pq2_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          GEMM_LDS_BYTES) == hipSuccess;
  if (!attr_ok) return -1;
  gemm_pq2_kernel<<<a.mt * a.nt, 256, GEMM_LDS_BYTES, st>>>(a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kq
