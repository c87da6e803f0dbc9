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
//   that is 512 tiles, two per CU, with no tail imbalance; the 128 x 80 wave
//   tile reads 208 operand rows from LDS per 10240 outputs, which keeps LDS
//   traffic under the MFMA time.
// * x' (bf16, from the rotation pre-pass) and the dequantized weight tile are
//   staged in LDS, double-buffered, rows padded to 72 bf16 so the 16-byte
//   operand reads of 16 rows are bank-conflict free.  The next K-tile is
//   fetched into registers while the current one is multiplied; one barrier
//   per K-tile.
// * Dequantization: 160 threads each expand the 64 codes of one weight row
//   per K-tile: fp4 conversion of the nibble-spread codes gives c exactly,
//   c*d - d is exact in fp32, and v_cvt_pk_bf16_f32 rounds pairs to bf16
//   (nearest even) -- the same value as (q-1) * bf16(d).
// * Tile order is XCD-aware: the 8 XCDs each take a contiguous eighth of the
//   token tiles and walk every weight tile over it, so the x' rows stay in
//   that XCD's L2 while the (ten times smaller) weight tiles stream past.
//   Ordered the other way round, every XCD streamed all of x' once per
//   weight tile it owned.
#include <type_traits>

#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int TM = 256, TN = 160, TK = 64;
constexpr int LDK = TK + 8;  // padded row stride (bf16 elements)
constexpr int TNS = 256;  // B rows staged per stage (rows past TN are padding, never read)
constexpr int STAGE_ELEMS = (TM + TNS) * LDK;
constexpr int GEMM_LDS_BYTES = 2 * STAGE_ELEMS * 2;  // 2 stages x (A + B) x bf16
constexpr int WM = TM / 2, WN = TN / 2;              // wave tile 128 x 80
constexpr int FM = WM / 16, FN = WN / 16;            // 8 x 5 MFMA tiles per wave

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

__device__ __forceinline__ void dequant_word_bf16(uint32_t w, float d, uint32_t* out8) {
  // 16 codes -> 16 bf16 values (q-1)*d, packed in 8 dwords (element order)
  const uint32_t e = w & 0x33333333u;
  const uint32_t o = (w >> 2) & 0x33333333u;
  float v[16];
  f32x2 t;
  t = codes2<0>(e); v[0] = t.x; v[2] = t.y;
  t = codes2<0>(o); v[1] = t.x; v[3] = t.y;
  t = codes2<1>(e); v[4] = t.x; v[6] = t.y;
  t = codes2<1>(o); v[5] = t.x; v[7] = t.y;
  t = codes2<2>(e); v[8] = t.x; v[10] = t.y;
  t = codes2<2>(o); v[9] = t.x; v[11] = t.y;
  t = codes2<3>(e); v[12] = t.x; v[14] = t.y;
  t = codes2<3>(o); v[13] = t.x; v[15] = t.y;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out8[i] = pack_bf16x2(fmaf(v[2 * i], d, -d), fmaf(v[2 * i + 1], d, -d));
}

__global__ __launch_bounds__(256, 1) void gemm_pq2_kernel(GemmArgs a) {
  extern __shared__ uint16_t smem[];
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

  // ---- global load geometry.  x' tile: load i of thread t covers row
  // 32 i + t / 8, bytes 16 (t % 8) .. +15 of its 128-byte K-tile slice, so
  // one instruction reads 8 whole rows.  Weights: thread t < TN expands the
  // 64 codes of row n0 + t.
  // All three go through buffer resources that cover exactly the block's
  // valid rows, so rows past M or N (and staging rows past TN) read zeros
  // with no branch: code 0 with scale 0 dequantizes to 0.
  const int arow = tid >> 3, achunk = (tid & 7) * 8;  // row in a group of 32, bf16 offset
  const int64_t G = a.d_per_row;
  const int64_t arows = a.M - m0 < TM ? a.M - m0 : TM;
  const int64_t brows = a.N - n0 < TN ? a.N - n0 : TN;
  const BufRsrc ra_rs = make_rsrc(a.xb + m0 * a.K, (uint32_t)(arows * a.K * 2));
  // codes of row n0 + t: tile (n0 + t) / 16 (n0 is a multiple of 16), row t % 16
  const BufRsrc rq_rs = make_rsrc(a.qs + (n0 >> 4) * G * 512, (uint32_t)((brows + 15) / 16 * G * 512));
  // scales of row n0 + t, block b: chunk ((n0 + t) / 16, b / 8), row t % 16
  const BufRsrc rd_rs = make_rsrc(a.dpl + (n0 >> 4) * a.d_tile_bytes, (uint32_t)((brows + 15) / 16 * a.d_tile_bytes));
  const uint32_t a_off = (uint32_t)(arow * a.K + achunk) * 2u;
  const uint32_t q_off = (uint32_t)((tid >> 4) * G * 512 + (tid & 15) * 32);
  const uint32_t d_off = (uint32_t)((tid >> 4) * a.d_tile_bytes + (tid & 15) * 16);

  // staging registers for two K-tiles: the tile stored during a K-tile's
  // multiplies was loaded one iteration earlier, so storing it never waits
  uint4 ra[2][8];
  uint4 rq[2];
  float rd[2];
  auto gload = [&](int kt, int set) {
    const int64_t k0 = (int64_t)kt * TK;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ra[set][i] = buffer_load_16B(ra_rs, a_off + (uint32_t)((32 * i * a.K + k0) * 2));
    rq[set] = buffer_load_16B(rq_rs, q_off + (uint32_t)((k0 >> 7) * 512 + ((k0 & 127) >> 2)));
    rd[set] = f16_bits_to_f32(buffer_load_2B(rd_rs, d_off + (uint32_t)((k0 >> 10) * 256 + ((k0 >> 7) & 7) * 2)));
  };
  auto sstore = [&](int buf, int set) {
    uint16_t* A = smem + buf * STAGE_ELEMS;
    uint16_t* B = A + TM * LDK;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(A + (32 * i + arow) * LDK + achunk) = ra[set][i];
    {
      uint32_t b8[32];
      dequant_word_bf16(rq[set].x, rd[set], b8);
      dequant_word_bf16(rq[set].y, rd[set], b8 + 8);
      dequant_word_bf16(rq[set].z, rd[set], b8 + 16);
      dequant_word_bf16(rq[set].w, rd[set], b8 + 24);
      uint4* pb = reinterpret_cast<uint4*>(B + tid * LDK);
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = make_uint4(b8[4 * i], b8[4 * i + 1], b8[4 * i + 2], b8[4 * i + 3]);
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int KT = (int)(a.K / TK);  // even: K is a multiple of 128
  gload(0, 0);
  gload(1, 1);
  sstore(0, 0);
  __syncthreads();

  // operand rows: lane (r, kq) reads 8 bf16 at k = 8 kq of row r of a 16-row tile
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  auto mma_tile = [&](int buf) {
    const uint16_t* A = smem + buf * STAGE_ELEMS + (wm * WM + fr) * LDK + fk;
    const uint16_t* B = smem + buf * STAGE_ELEMS + TM * LDK + (wn * WN + fr) * LDK + fk;
#pragma unroll
    for (int ks = 0; ks < TK / 32; ++ks) {
      bf16x8 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(A + i * 16 * LDK + ks * 32);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(B + j * 16 * LDK + ks * 32);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  // K-tile kt: multiply buffer kt % 2, store tile kt + 1 (staged in set
  // (kt + 1) % 2) into the other buffer, load tile kt + 2 into set kt % 2.
  // Unrolled by two so buffer and set indices are compile-time constants.
  // steady state: load, multiply and store in one basic block, with the
  // staging work (code and x' loads, dequantization, LDS writes) interleaved
  // between the MFMAs: each MFMA is followed by two vector-ALU slots, the
  // second k-step's fragment reads ride on the first 13, the LDS writes on
  // the second 16
  auto step = [&](int kt, auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    gload(kt + 2, buf);
    mma_tile(buf);
    sstore(buf ^ 1, buf ^ 1);
    __builtin_amdgcn_sched_group_barrier(0x020, 10, 0);  // global loads
    __builtin_amdgcn_sched_group_barrier(0x100, 13, 0);  // fragment reads, k-step 0
#pragma unroll
    for (int i = 0; i < 40; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      if (i < 13) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 40; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      if (i < 16) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 3 < KT; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
  }
  // last two K-tiles (KT is even): store the final tile, then multiply it
  mma_tile(0);
  sstore(1, 1);
  __syncthreads();
  mma_tile(1);

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
