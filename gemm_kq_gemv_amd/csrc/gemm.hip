// gemm.hip -- PQ2_0 prefill GEMM on bf16 MFMA.
//
// y[m][n] = sum_k bf16((q-1)*d)[n][k] * bf16(x'[m][k]), fp32 accumulation.
// Each weight block is dequantized once per LDS tile and the tile is reused
// by every token row of the workgroup (the dequantize-once-per-tile prefill
// scheme of the Kipp Benchmarks page, "Quantized projections on the tensor
// units"; the Bonsai page's tiled ternary GEMM, sec. 8.3, 8.5).
//
// gfx950 design (v1)
// ------------------
// * Tile 128 (tokens) x 128 (weight rows) x 64 (K) per workgroup of 4
//   waves; each wave owns a 64 x 64 sub-tile = 2 x 2 v_mfma_f32_32x32x16_bf16
//   accumulators (64 fp32 registers).
// * x' (bf16, produced by the Hadamard pre-pass) and the dequantized weight
//   tile are staged in LDS, double-buffered, rows padded to 72 bf16 so the
//   MFMA operand reads (16 B per lane, 32 rows) are bank-conflict free.  The
//   next K-tile is fetched into registers while the current one is
//   multiplied; one barrier per K-tile.
// * Dequantization: one thread expands 32 codes of one row per K-tile:
//   fp4 conversion of the nibble-spread codes gives c exactly, c*d - d is
//   exact in fp32, and v_cvt_pk_bf16_f32 rounds pairs to bf16 (nearest even)
//   -- the same value as (q-1) * bf16(d).
// * Tile order is XCD-aware: the 8 XCDs each take a contiguous eighth of the
//   weight-row tiles and walk all token tiles over it, so a weight tile stays
//   in that XCD's L2 while the token tiles stream past.
#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDA = BK + 8;  // padded row stride (bf16 elements)
constexpr int TILE_ELEMS = 128 * LDA;
constexpr int GEMM_LDS_BYTES = 2 * 2 * TILE_ELEMS * 2;  // 2 buffers x (A + B) x bf16

struct GemmArgs {
  const uint16_t* xb;   // x' bf16 [M][K]
  const uint8_t* qs;    // qs plane
  const uint16_t* dpl;  // d plane
  float* y;             // [M][N]
  int64_t M, N, K;
  int64_t row_bytes, d_per_row;
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

__global__ __launch_bounds__(256, 2) void gemm_pq2_kernel(GemmArgs a) {
  extern __shared__ uint16_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- XCD-aware tile mapping
  const int bid = blockIdx.x;
  int m_tile, n_tile;
  if ((a.nt & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3;
    const int npx = a.nt >> 3;
    n_tile = xcd * npx + local % npx;
    m_tile = local / npx;
  } else {
    n_tile = bid % a.nt;
    m_tile = bid / a.nt;
  }
  const int64_t m0 = (int64_t)m_tile * BM, n0 = (int64_t)n_tile * BN;

  // ---- per-thread global load geometry: row tid/2, half tid&1
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t am = m0 + lr, bn = n0 + lr;
  const bool a_ok = am < a.M, b_ok = bn < a.N;
  const uint16_t* a_src = a.xb + am * a.K + lh * 32;
  // codes of row bn: tile (bn / 16, k / 128), row bn % 16 at 32 bytes each
  const uint8_t* b_src = a.qs + (bn >> 4) * (a.d_per_row * 512) + (bn & 15) * 32 + lh * 8;
  const uint16_t* d_src = a.dpl + bn * a.d_per_row;

  uint4 ra[4];
  uint2 rq;
  float rd;
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    if (a_ok) {
      const uint4* p = reinterpret_cast<const uint4*>(a_src + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (b_ok) {
      rq = *reinterpret_cast<const uint2*>(b_src + (k0 >> 7) * 512 + ((k0 & 127) >> 2));
      rd = f16_bits_to_f32(d_src[k0 >> 7]);
    } else {
      rq = make_uint2(0x55555555u, 0x55555555u);
      rd = 0.f;
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* A = smem + buf * 2 * TILE_ELEMS;
    uint16_t* B = A + TILE_ELEMS;
    uint4* pa = reinterpret_cast<uint4*>(A + lr * LDA + lh * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) pa[i] = ra[i];
    uint32_t b8[16];
    dequant_word_bf16(rq.x, rd, b8);
    dequant_word_bf16(rq.y, rd, b8 + 8);
    uint4* pb = reinterpret_cast<uint4*>(B + lr * LDA + lh * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = make_uint4(b8[4 * i], b8[4 * i + 1], b8[4 * i + 2], b8[4 * i + 3]);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (int)(a.K / BK);
  gload(0);
  sstore(0);
  __syncthreads();

  const int ar = lane & 31, ak = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint16_t* A = smem + buf * 2 * TILE_ELEMS;
    const uint16_t* B = A + TILE_ELEMS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(A + (wm * 64 + i * 32 + ar) * LDA + ks * 16 + ak);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(B + (wn * 64 + j * 32 + ar) * LDA + ks * 16 + ak);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
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
  a.dpl = (const uint16_t*)pv.d;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  a.row_bytes = pv.row_bytes;
  a.d_per_row = pv.d_per_row;
  a.mt = (int)((M + BM - 1) / BM);
  a.nt = (int)((N + BN - 1) / BN);
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
