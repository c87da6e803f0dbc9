// gemv.hip -- quantized GEMV (M = 1..8 activation rows), PQ2_0 and Q8_0.
//
// y[m][n] = sum_k deq(W)[n][k] * x'[m][k]
//   PQ2_0 deq = (q-1)*d per 128-group (Bonsai ternary g128 page, sec. 3.1);
//   Q8_0  deq = d*q per 32-group (Kipp pages).
//
// gfx950 design
// -------------
// * Work unit.  A row of the qs plane is cut into 16-byte chunks (64 PQ2_0
//   codes or 16 Q8_0 weights; both are half a quantization group, so a chunk
//   has exactly one scale).  A wavefront owns a contiguous run of rows and
//   walks them in batches of RB rows.  One "step" loads one chunk per lane
//   for each of the RB rows: lane l takes chunk p*64 + l, so every load
//   instruction is a fully coalesced 1 KiB dwordx4 read of one row.  When the
//   chunk count is not a multiple of 64, the remaining T chunks are covered
//   by a tail step in which the wave is split into G = 64/T lane groups that
//   each take a different row (no idle lanes when T divides 64).
// * Latency.  The loads of step s+1 are issued before step s is computed, so
//   a wave always has one step of loads in flight; the launch gives every
//   SIMD an equal number of rows (two waves per SIMD), which matters because
//   the PQ2_0 decode keeps the VALU nearly as busy as HBM.
// * Activation.  The workgroup stages its K-range of x' (fp32) in LDS once;
//   each chunk is padded by 16 bytes so that the 64 lanes' dwordx4 LDS reads
//   hit distinct banks.  A lane re-reads x' per step, amortised over RB rows.
// * PQ2_0 decode.  (w & 0x33333333) and ((w >> 2) & 0x33333333) leave one
//   2-bit code in each nibble; the gfx950 fp4 converter turns two nibbles
//   into two exact floats (scale 2 gives the code c itself), so 16 codes cost
//   3 bit ops + 8 conversions + 16 FMAs.  The ternary map's -1 is folded into
//   a per-chunk activation sum X computed at staging time:
//   sum (c-1) x' = sum c x' - X   (the Bonsai page, sec. 8.5, folds the -1
//   the same way).
// * Q8_0 decode.  Each int8 is converted with a sign-extending byte select
//   (one instruction per weight).
// * Reduction.  Per row, the 64 lane partials are summed with DPP row
//   reductions plus four lane reads (fixed order, deterministic); tail-step
//   partials go through a small per-wave LDS scratch and are summed by the
//   row's owning lane in lane order.  fp32 throughout; no atomics.
// * Split-K.  blockIdx.y selects one of S contiguous ranges of whole groups;
//   each range writes fp32 partials [S][M][N] that a second kernel adds in
//   ascending s.
#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

constexpr int kWavesPerGroup = 4;
constexpr int kPad = 4;  // floats of padding per staged chunk

template <int FMT>
struct Fmt;
template <>
struct Fmt<kFmtPQ2> {
  static constexpr int CW = 64;   // activation floats per 16-byte chunk
  static constexpr int VPW = 16;  // values per 32-bit word
  static constexpr bool FOLD = true;
};
template <>
struct Fmt<kFmtQ8> {
  static constexpr int CW = 16;
  static constexpr int VPW = 4;
  static constexpr bool FOLD = false;
};

template <int M>
struct RowsPerBatch {
  static constexpr int value = M <= 2 ? 8 : (M <= 4 ? 4 : 2);
};

struct GemvArgs {
  const uint8_t* qs;
  const uint16_t* dpl;
  const float* xr;  // x' [M][K] fp32
  float* out;       // y [M][N] (S == 1) or partials [S][M][N]
  int64_t N, K;
  int64_t row_bytes;  // qs bytes per row
  int64_t d_per_row;
  int n_groups;       // quantization groups per row
  int split;          // S
  int rows_per_wave;
  int max_slice_chunks;  // LDS is sized for this many chunks
};

// Decode one 32-bit word into VPW floats.
template <int FMT>
__device__ __forceinline__ void decode_word(uint32_t w, float* v);

template <>
__device__ __forceinline__ void decode_word<kFmtPQ2>(uint32_t w, float* v) {
  const uint32_t e = w & 0x33333333u;         // codes 0,2,4,..,14 (one per nibble)
  const uint32_t o = (w >> 2) & 0x33333333u;  // codes 1,3,5,..,15
  f32x2 a;
  a = codes2<0>(e); v[0] = a.x; v[2] = a.y;
  a = codes2<0>(o); v[1] = a.x; v[3] = a.y;
  a = codes2<1>(e); v[4] = a.x; v[6] = a.y;
  a = codes2<1>(o); v[5] = a.x; v[7] = a.y;
  a = codes2<2>(e); v[8] = a.x; v[10] = a.y;
  a = codes2<2>(o); v[9] = a.x; v[11] = a.y;
  a = codes2<3>(e); v[12] = a.x; v[14] = a.y;
  a = codes2<3>(o); v[13] = a.x; v[15] = a.y;
}

template <>
__device__ __forceinline__ void decode_word<kFmtQ8>(uint32_t w, float* v) {
  v[0] = (float)(int8_t)(w);
  v[1] = (float)(int8_t)(w >> 8);
  v[2] = (float)(int8_t)(w >> 16);
  v[3] = (float)(int8_t)(w >> 24);
}

template <int FMT, int M>
__global__ __launch_bounds__(256, 2) void gemv_kernel(GemvArgs a) {
  using F = Fmt<FMT>;
  constexpr int CW = F::CW;
  constexpr int CS = CW + kPad;  // staged chunk stride (floats)
  constexpr int RB = RowsPerBatch<M>::value;
  extern __shared__ float lds[];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;

  // ---- K range of this slice (whole groups), in chunks (2 per group)
  const int s = blockIdx.y;
  const int g0 = (int)((int64_t)s * a.n_groups / a.split);
  const int g1 = (int)((int64_t)(s + 1) * a.n_groups / a.split);
  const int c0 = 2 * g0;
  const int Cs = 2 * (g1 - g0);
  const int Qs = Cs >> 6;   // full main passes
  const int Ts = Cs & 63;   // tail chunks
  const int G = Ts ? (64 / Ts) : 1;           // rows per tail load
  const int RBt = Ts ? (RB + G - 1) / G : 0;  // tail loads per batch
  const int steps_per_batch = Qs + (Ts ? 1 : 0);

  // ---- rows of this wave
  const int64_t wave_id = (int64_t)blockIdx.x * kWavesPerGroup + wave;
  const int64_t r_begin = wave_id * a.rows_per_wave;
  const int64_t r_end = r_begin + a.rows_per_wave < a.N ? r_begin + a.rows_per_wave : a.N;
  const int n_batches = r_begin < r_end ? (int)((r_end - r_begin + RB - 1) / RB) : 0;
  const int n_steps = n_batches * steps_per_batch;

  float* xs = lds;                                        // [M][Cs][CS]
  float* xsum = lds + M * a.max_slice_chunks * CS;        // [M][Cs] (PQ2_0)
  float* scratch = xsum + (F::FOLD ? M * a.max_slice_chunks : 0) +
                   wave * (RB * M * 64);                  // per-wave tail scratch

  // step s -> (row0, pass) ; per-lane load geometry
  const int tail_row = Ts ? lane / Ts : 0;
  const int tail_chunk = Ts ? (Qs << 6) + lane % Ts : 0;
  const bool tail_lane = Ts ? lane < G * Ts : false;

  uint4 cq[RB], nq[RB];
  float cd[RB], nd[RB];

  auto load_step = [&](int step, uint4* q, float* d) {
    const int b = step / steps_per_batch;
    const int p = step - b * steps_per_batch;
    const int64_t row0 = r_begin + (int64_t)b * RB;
    const bool tail = p == Qs;
    const int chunk = tail ? tail_chunk : (p << 6) + lane;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int64_t row = tail ? row0 + (int64_t)G * j + tail_row : row0 + j;
      const bool ok = tail ? (j < RBt && tail_lane && row < r_end && row < row0 + RB)
                           : (row < r_end);
      if (ok) {
        q[j] = *reinterpret_cast<const uint4*>(a.qs + row * a.row_bytes + (int64_t)(c0 + chunk) * 16);
        d[j] = f16_bits_to_f32(a.dpl[row * a.d_per_row + ((c0 + chunk) >> 1)]);
      } else {
        q[j] = make_uint4(0u, 0u, 0u, 0u);
        d[j] = 0.f;
      }
    }
  };

  // Issue the first step's weight loads before staging x' so that their
  // latency overlaps the staging.
  if (n_steps > 0) load_step(0, cq, cd);

  // ---- stage x'[m][c0*CW, (c0+Cs)*CW) into LDS
  {
    const int f4_per_chunk = CW / 4;
    const int total = M * Cs * f4_per_chunk;
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
      const int m = i / (Cs * f4_per_chunk);
      const int r = i - m * Cs * f4_per_chunk;
      const int c = r / f4_per_chunk;
      const int q = r - c * f4_per_chunk;
      const float4 v = *reinterpret_cast<const float4*>(a.xr + (int64_t)m * a.K + (int64_t)(c0 + c) * CW + 4 * q);
      *reinterpret_cast<float4*>(xs + (m * a.max_slice_chunks + c) * CS + 4 * q) = v;
    }
  }
  __syncthreads();
  if (F::FOLD) {
    for (int i = threadIdx.x; i < M * Cs; i += blockDim.x) {
      const int m = i / Cs, c = i - m * Cs;
      const float* p = xs + (m * a.max_slice_chunks + c) * CS;
      float t = 0.f;
      for (int j = 0; j < CW; ++j) t += p[j];
      xsum[m * a.max_slice_chunks + c] = t;
    }
    __syncthreads();
  }

  float acc[RB][M], tacc[RB][M];
#pragma unroll
  for (int j = 0; j < RB; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[j][m] = tacc[j][m] = 0.f;

  for (int step = 0; step < n_steps; ++step) {
    const int b = step / steps_per_batch;
    const int p = step - b * steps_per_batch;
    const bool tail = p == Qs;
    const int64_t row0 = r_begin + (int64_t)b * RB;
    const int rows_here = (int)(r_end - row0 < RB ? r_end - row0 : RB);

    if (step + 1 < n_steps) load_step(step + 1, nq, nd);

    // ---- compute this step
    const int chunk = tail ? tail_chunk : (p << 6) + lane;
    const bool lane_ok = tail ? tail_lane : true;
    const int nloads = tail ? RBt : rows_here;
    float S[RB][M];
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int m = 0; m < M; ++m) S[j][m] = 0.f;

    if (lane_ok) {
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        float xv[M][F::VPW];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float* src = xs + (m * a.max_slice_chunks + chunk) * CS + wi * F::VPW;
#pragma unroll
          for (int i = 0; i < F::VPW; i += 4) {
            const float4 t = *reinterpret_cast<const float4*>(src + i);
            xv[m][i] = t.x; xv[m][i + 1] = t.y; xv[m][i + 2] = t.z; xv[m][i + 3] = t.w;
          }
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          if (j < nloads) {
            const uint32_t w = wi == 0 ? cq[j].x : wi == 1 ? cq[j].y : wi == 2 ? cq[j].z : cq[j].w;
            float v[F::VPW];
            decode_word<FMT>(w, v);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
              for (int i = 0; i < F::VPW; ++i) S[j][m] = fmaf(v[i], xv[m][i], S[j][m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float X = F::FOLD ? xsum[m * a.max_slice_chunks + chunk] : 0.f;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const float t = F::FOLD ? (S[j][m] - X) : S[j][m];
          if (tail)
            tacc[j][m] = fmaf(cd[j], t, tacc[j][m]);
          else
            acc[j][m] = fmaf(cd[j], t, acc[j][m]);
        }
      }
    }

    // ---- end of a batch: reduce and store
    if (p == steps_per_batch - 1) {
      float mine[M];
#pragma unroll
      for (int m = 0; m < M; ++m) mine[m] = 0.f;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (j < rows_here) {
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float tot = wave_sum(acc[j][m]);
            mine[m] = lane == j ? tot : mine[m];
          }
        }
      }
      if (Ts) {
        // tail partials: lane l of tail load j holds row G*j + l/Ts
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
          for (int m = 0; m < M; ++m) scratch[(j * M + m) * 64 + lane] = tacc[j][m];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < rows_here) {
          const int jt = lane / G, gt = lane - jt * G;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float* src = scratch + (jt * M + m) * 64 + gt * Ts;
            float t = 0.f;
            for (int i = 0; i < Ts; ++i) t += src[i];
            mine[m] += t;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      if (lane < rows_here) {
        float* o = a.out + (int64_t)s * M * a.N + row0 + lane;
#pragma unroll
        for (int m = 0; m < M; ++m) o[(int64_t)m * a.N] = mine[m];
      }
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[j][m] = tacc[j][m] = 0.f;
    }

#pragma unroll
    for (int j = 0; j < RB; ++j) { cq[j] = nq[j]; cd[j] = nd[j]; }
  }
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

static int rows_per_batch(int64_t M) { return M <= 2 ? 8 : (M <= 4 ? 4 : 2); }
static constexpr int kLdsBudget = 64 * 1024;
static constexpr int kTargetWaves = 2048;  // 256 CUs x 4 SIMDs x 2

static int64_t lds_bytes_for(int fmt, int64_t M, int chunks) {
  const int CW = fmt == kFmtPQ2 ? 64 : 16;
  int64_t b = M * chunks * (CW + kPad) * 4;
  if (fmt == kFmtPQ2) b += M * chunks * 4;
  b += (int64_t)kWavesPerGroup * rows_per_batch(M) * M * 64 * 4;
  return b;
}

GemvPlan plan_gemv(int fmt, int64_t M, int64_t N, int64_t K, int split_req) {
  GemvPlan p{};
  const int n_groups = (int)(K / group_of(fmt));
  int s_min = 1;
  while (s_min <= n_groups &&
         lds_bytes_for(fmt, M, 2 * ((n_groups + s_min - 1) / s_min)) > kLdsBudget)
    ++s_min;
  int S = split_req > 0 ? split_req : s_min;
  if (S > n_groups || S < s_min) { p.split = -1; return p; }
  p.split = S;
  const int max_chunks = 2 * ((n_groups + S - 1) / S);
  p.lds_bytes = (int)lds_bytes_for(fmt, M, max_chunks);
  int64_t waves = kTargetWaves / S;
  if (waves < kWavesPerGroup) waves = kWavesPerGroup;
  int64_t rpw = (N + waves - 1) / waves;
  if (rpw < 1) rpw = 1;
  p.rows_per_wave = (int)rpw;
  int64_t w_needed = (N + rpw - 1) / rpw;
  p.grid_x = (int)((w_needed + kWavesPerGroup - 1) / kWavesPerGroup);
  return p;
}

int64_t gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int block_len,
                             int split_req) {
  (void)block_len;
  GemvPlan p = plan_gemv(fmt, M, N, K, split_req);
  if (p.split < 1) return -1;
  int64_t b = (M * K * 4 + 255) / 256 * 256;  // x'
  if (p.split > 1) b += (int64_t)p.split * M * N * 4;
  return b;
}

template <int FMT, int M>
static void launch_one(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  dim3 grid(p.grid_x, p.split);
  gemv_kernel<FMT, M><<<grid, kWavesPerGroup * 64, p.lds_bytes, st>>>(a);
}

template <int FMT>
static void launch_fmt(int64_t M, const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  switch (M) {
    case 1: launch_one<FMT, 1>(a, p, st); break;
    case 2: launch_one<FMT, 2>(a, p, st); break;
    case 3: launch_one<FMT, 3>(a, p, st); break;
    case 4: launch_one<FMT, 4>(a, p, st); break;
    case 5: launch_one<FMT, 5>(a, p, st); break;
    case 6: launch_one<FMT, 6>(a, p, st); break;
    case 7: launch_one<FMT, 7>(a, p, st); break;
    default: launch_one<FMT, 8>(a, p, st); break;
  }
}

int launch_gemv(int fmt, const void* packed, int64_t N, int64_t K, const float* x, int64_t M,
                int block_len, const int8_t* signs, int split_req, float* y, void* ws,
                hipStream_t st) {
  GemvPlan p = plan_gemv(fmt, M, N, K, split_req);
  if (p.split < 1) return -2;
  const float* xr = x;
  float* xprime = (float*)ws;
  if (block_len > 0 || signs) {
    if (launch_hadamard(x, 0, xprime, 0, M, K, block_len > 0 ? block_len : 1, signs, st)) return -1;
    xr = xprime;
  }
  PlanarView pv = planar_view(fmt, N, K, const_cast<void*>(packed));
  GemvArgs a;
  a.qs = pv.qs;
  a.dpl = (const uint16_t*)pv.d;
  a.xr = xr;
  a.N = N;
  a.K = K;
  a.row_bytes = pv.row_bytes;
  a.d_per_row = pv.d_per_row;
  a.n_groups = (int)(K / group_of(fmt));
  a.split = p.split;
  a.rows_per_wave = p.rows_per_wave;
  a.max_slice_chunks = 2 * ((a.n_groups + p.split - 1) / p.split);
  float* part = nullptr;
  if (p.split > 1) {
    part = (float*)((uint8_t*)ws + (M * K * 4 + 255) / 256 * 256);
    a.out = part;
  } else {
    a.out = y;
  }
  if (fmt == kFmtPQ2)
    launch_fmt<kFmtPQ2>(M, a, p, st);
  else
    launch_fmt<kFmtQ8>(M, a, p, st);
  if (hipGetLastError() != hipSuccess) return -1;
  if (p.split > 1) {
    int64_t n = M * N;
    splitk_reduce_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(part, y, n, p.split);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace kq
