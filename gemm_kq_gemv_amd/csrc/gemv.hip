// gemv.hip -- quantized GEMV (M = 1..8 activation rows), PQ2_0 and Q8_0.
//
// y[m][n] = sum_k deq(W)[n][k] * x'[m][k],   x' = blockwise rotation of x
//   PQ2_0 deq = (q-1)*d per 128-group (Bonsai ternary g128 page, sec. 3.1);
//   Q8_0  deq = d*q per 32-group (Kipp pages);
//   x' = (1/sqrt(n)) H_n (s (.) x) per n-block (Bonsai page, sec. 4.1-4.2).
//
// gfx950 design
// -------------
// * One launch.  Every workgroup (8 waves, one per CU) first turns its
//   K-range of x into x' in LDS -- sign flip, in-register and cross-lane
//   butterflies, 1/sqrt(n) -- so the rotation costs no extra kernel launch
//   and x' never goes through memory.
// * Work unit.  A row of the qs plane is cut into 16-byte chunks (64 PQ2_0
//   codes or 16 Q8_0 weights; half a quantization group each, so a chunk has
//   one scale).  A wave owns a contiguous run of rows and walks them in
//   batches of RB rows.  One "step" loads one chunk per lane for each of the
//   RB rows: lane l takes chunk p*64 + l, so each load instruction is a
//   coalesced 1 KiB dwordx4 read of one row.  The T chunks left when a row is
//   not a multiple of 64 chunks form a tail step in which the wave splits
//   into G = 64/T lane groups, one row each.
// * Loads.  Buffer loads whose resource covers exactly the batch's rows: rows
//   past the batch or past N and the idle lanes of a tail step read zeros
//   from the hardware range check, so the loads need no branches and the
//   loads of step s+2 stay in flight while step s is computed (three
//   rotating register buffers).  Every SIMD gets the same number of rows.
// * PQ2_0 arithmetic.  x' is staged as fp16 pairs: each 128-element group of
//   x' is scaled by a power of two that puts its largest magnitude in
//   [2^14, 2^15) (the inverse is folded into the weight scale), then rounded
//   once to fp16 -- the activation precision of the pages' own matvec
//   kernels -- so each product is exact to 2^-11 relative and the result
//   stays within 2^-11 * sum|W x'| plus fp32 accumulation error.
//   (w & 0x33333333) and ((w >> 2) & 0x33333333) leave one 2-bit code per
//   nibble; the gfx950 fp4 converter turns two nibbles into an exact fp16
//   pair (scale 2 gives the code c), and v_dot2_f32_f16 multiplies it with
//   the matching x' pair, accumulating in fp32: 16 codes cost 3 bit ops +
//   8 conversions + 8 dot products.  The ternary map's -1 is folded into a
//   per-chunk sum X of the same fp16 values:
//   sum (c-1) x' = sum c x' - X   (the Bonsai page, sec. 8.5, folds the -1
//   the same way).
// * Q8_0 arithmetic.  x' stays fp32; each int8 is converted with a
//   sign-extending byte select and multiplied with an fp32 FMA.
// * Reduction.  Per row, the 64 lane partials are summed with DPP row
//   reductions plus four lane reads (fixed order, deterministic); tail-step
//   partials go through a small per-wave LDS scratch and are summed by the
//   row's owning lane in lane order.  No atomics.
// * Split-K.  blockIdx.y selects one of S contiguous ranges of whole groups;
//   each range writes fp32 partials [S][M][N] that a second kernel adds in
//   ascending s.
#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

constexpr int kWaves = 8;  // waves per workgroup (one workgroup per CU)
constexpr int kThreads = kWaves * 64;
constexpr int kPadDW = 4;  // dwords of padding per staged chunk (bank spread)

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int FMT>
struct Fmt;
template <>
struct Fmt<kFmtPQ2> {
  static constexpr int CW = 64;        // elements per 16-byte chunk
  static constexpr int CHUNK_DW = 32;  // staged dwords per chunk (fp16 pairs)
  static constexpr int XDW = 8;        // staged dwords per 32-bit weight word
  static constexpr bool FOLD = true;
};
template <>
struct Fmt<kFmtQ8> {
  static constexpr int CW = 16;
  static constexpr int CHUNK_DW = 16;  // fp32
  static constexpr int XDW = 4;
  static constexpr bool FOLD = false;
};

template <int M>
struct RowsPerBatch {
  static constexpr int value = M <= 2 ? 8 : (M <= 4 ? 4 : 2);
};

struct GemvArgs {
  const uint8_t* qs;
  const uint16_t* dpl;
  const float* x;        // activations [M][K]: raw (rotated in the prologue) or x'
  const int8_t* signs;   // K entries applied in the prologue, or null
  float* out;            // y [M][N] (S == 1) or partials [S][M][N]
  int64_t N, K;
  int row_bytes;         // qs bytes per row
  int d_per_row;         // scales per row
  int n_groups;          // quantization groups per row
  int split;             // S
  int rows_per_wave;
  int max_slice_chunks;  // LDS is sized for this many chunks
  int log2n;             // butterfly stages of the prologue rotation (0: none)
  float scale;           // 1/sqrt(n), or 1
};

// two 2-bit codes (one per nibble of byte SEL) -> exact fp16 pair (c, c')
template <int SEL>
__device__ __forceinline__ f16x2 codes2h(uint32_t spread) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(spread, 2.0f, SEL);
}

__device__ __forceinline__ float dot2(f16x2 a, uint32_t b_bits, float c) {
  return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(f16x2, b_bits), c, false);
}

template <int FMT, int M>
__global__ __launch_bounds__(kThreads, 1) void gemv_kernel(GemvArgs a) {
  using F = Fmt<FMT>;
  constexpr int CW = F::CW;
  constexpr int CS = F::CHUNK_DW + kPadDW;  // staged chunk stride (dwords)
  constexpr int RB = RowsPerBatch<M>::value;
  extern __shared__ uint32_t lds[];

  const int lane = lane_id();
  // wave index as a scalar: everything derived from it (rows, buffer
  // resources) stays in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

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
  const int64_t wave_id = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t r_begin = wave_id * a.rows_per_wave;
  const int64_t r_end = r_begin + a.rows_per_wave < a.N ? r_begin + a.rows_per_wave : a.N;
  const int n_batches = r_begin < r_end ? (int)((r_end - r_begin + RB - 1) / RB) : 0;
  const int n_steps = n_batches * steps_per_batch;

  const int MC = a.max_slice_chunks;
  uint32_t* xs = lds;                                        // [M][MC][CS] staged x'
  float* xsum = reinterpret_cast<float*>(lds + M * MC * CS);  // [M][MC] chunk sums X
  float* xinv = xsum + (F::FOLD ? M * MC : 0);                // [M][MC] inverse range scale
  float* scratch = xinv + (F::FOLD ? M * MC : 0) + wave * (RB * M * 64);  // tail partials

  const int tail_row = Ts ? lane / Ts : 0;
  const int tail_chunk = Ts ? (Qs << 6) + lane % Ts : 0;
  const bool tail_lane = Ts ? lane < G * Ts : false;

  // Weight loads: branch-free buffer loads; the resource of a batch covers
  // exactly its rows of this K-slice.  Offsets are 32-bit: per lane a base,
  // plus a uniform row stride per load.
  const uint32_t rbytes = (uint32_t)a.row_bytes;
  const uint32_t dbytes = (uint32_t)a.d_per_row * 2u;
  // tail step: lane group tail_row takes rows tail_row, tail_row + G, ...
  const uint32_t tq_lane = tail_lane ? (uint32_t)tail_chunk * 16u + (uint32_t)tail_row * rbytes : kOutOfRange;
  const uint32_t td_lane = tail_lane ? (uint32_t)(tail_chunk >> 1) * 2u + (uint32_t)tail_row * dbytes : kOutOfRange;
  auto load_step = [&](int step, uint4 (&q)[RB], uint32_t (&d)[RB]) {
    const int b = step / steps_per_batch;
    const int p = step - b * steps_per_batch;
    const int64_t row0 = r_begin + (int64_t)b * RB;
    const int rows = (int)(r_end - row0 < RB ? r_end - row0 : RB);
    const BufRsrc rq = make_rsrc(a.qs + row0 * a.row_bytes + (int64_t)c0 * 16,
                                 (uint32_t)(rows - 1) * rbytes + (uint32_t)Cs * 16u);
    const BufRsrc rd = make_rsrc(a.dpl + row0 * a.d_per_row + g0,
                                 (uint32_t)(rows - 1) * dbytes + (uint32_t)(Cs >> 1) * 2u);
    if (p != Qs) {  // main step: lane takes chunk p*64 + lane of rows 0..RB-1
      const uint32_t q_lane = (uint32_t)((p << 6) + lane) * 16u;
      const uint32_t d_lane = (uint32_t)((p << 5) + (lane >> 1)) * 2u;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        q[j] = buffer_load_16B(rq, q_lane + (uint32_t)j * rbytes);
        d[j] = buffer_load_2B(rd, d_lane + (uint32_t)j * dbytes);  // raw fp16 bits
      }
    } else {        // tail step: load j takes row G*j + tail_row
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const bool ok = j < RBt;
        q[j] = buffer_load_16B(rq, ok ? tq_lane + (uint32_t)(G * j) * rbytes : kOutOfRange);
        d[j] = buffer_load_2B(rd, ok ? td_lane + (uint32_t)(G * j) * dbytes : kOutOfRange);
      }
    }
  };

  // ---- prologue: x -> x' in LDS.  Each thread owns 16 consecutive elements
  // of one row of the slice per iteration; an n-block (n <= 1024) is n/16
  // consecutive lanes of one wave.
  const int Ks = Cs * CW;
  const int g16_row = Ks >> 4;
  const int G16 = M * g16_row;
  const int iters = (G16 + kThreads - 1) / kThreads;
  auto load_group = [&](int it, float (&v)[16], uint4& sg) {
    const int gi = (int)threadIdx.x + it * kThreads;
    if (gi < G16) {
      const int m = gi / g16_row;
      const int64_t k = (int64_t)c0 * CW + (int64_t)(gi - m * g16_row) * 16;
      const float4* src = reinterpret_cast<const float4*>(a.x + (int64_t)m * a.K + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
      sg = a.signs ? *reinterpret_cast<const uint4*>(a.signs + k) : make_uint4(0u, 0u, 0u, 0u);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.f;
      sg = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto stage_group = [&](int it, float (&v)[16], const uint4& sg) {
    const int gi = (int)threadIdx.x + it * kThreads;
    const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
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
            const float p = v[i], q = v[i + h];
            v[i] = p + q;
            v[i + h] = p - q;
          }
      }
    }
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      if (st + 4 < a.log2n) {
        const int h = 1 << st;
        const bool upper = (lane & h) != 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __shfl_xor(v[i], h);
          v[i] = upper ? (p - v[i]) : (v[i] + p);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= a.scale;
    const bool live = gi < G16;
    const int m = live ? gi / g16_row : 0;
    const int e0 = live ? (gi - m * g16_row) * 16 : 0;
    const int c = e0 / CW;
    uint32_t* dst = xs + (m * MC + c) * CS + (e0 % CW) * F::CHUNK_DW / CW;
    if (F::FOLD) {
      // power-of-two range scale of the 128-element group (8 lanes)
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[i]));
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      int E = (int)((__float_as_uint(mx) >> 23) & 0xFFu);
      E = E < 15 ? 15 : (E > 254 ? 254 : E);
      const float sc = __uint_as_float((uint32_t)(268 - E) << 23);   // 2^(141-E)
      const float inv = __uint_as_float((uint32_t)(E - 14) << 23);   // 2^(E-141)
      // fp16 pairs in decode order: (0,2) (1,3) (4,6) (5,7) ...
      uint32_t h[8];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f16x2 pe = {(_Float16)(v[4 * b] * sc), (_Float16)(v[4 * b + 2] * sc)};
        const f16x2 po = {(_Float16)(v[4 * b + 1] * sc), (_Float16)(v[4 * b + 3] * sc)};
        h[2 * b] = __builtin_bit_cast(uint32_t, pe);
        h[2 * b + 1] = __builtin_bit_cast(uint32_t, po);
      }
      // X = sum of the staged fp16 values (same dot2 arithmetic as the codes)
      const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) part = dot2(ones, h[i], part);
      part += __shfl_xor(part, 1);  // a 64-element chunk is 4 consecutive lanes
      part += __shfl_xor(part, 2);
      if (live) {
        uint4* d4 = reinterpret_cast<uint4*>(dst);
        d4[0] = make_uint4(h[0], h[1], h[2], h[3]);
        d4[1] = make_uint4(h[4], h[5], h[6], h[7]);
        if ((gi & 3) == 0) {
          xsum[m * MC + c] = part;
          xinv[m * MC + c] = inv;
        }
      }
    } else if (live) {
      uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        d4[i] = make_uint4(__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                           __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3]));
    }
  };

  uint4 q0[RB], q1[RB], q2[RB];
  uint32_t d0[RB], d1[RB], d2[RB];
  {
    float v[16];
    uint4 sg;
    // activation loads first, then the first two weight steps, so that the
    // prologue only waits for the (small) activation loads
    // waves with no element in an iteration skip it (uniform; the shuffles
    // never leave a wave)
    const int wave_first = __builtin_amdgcn_readfirstlane((int)(threadIdx.x & ~63u));
    load_group(0, v, sg);
    if (n_steps > 0) load_step(0, q0, d0);
    if (n_steps > 1) load_step(1, q1, d1);
    if (wave_first < G16) stage_group(0, v, sg);
    for (int it = 1; it < iters; ++it) {
      load_group(it, v, sg);
      if (wave_first + it * kThreads < G16) stage_group(it, v, sg);
    }
  }
  __syncthreads();

  float acc[RB][M], tacc[RB][M];
#pragma unroll
  for (int j = 0; j < RB; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[j][m] = tacc[j][m] = 0.f;

  auto body = [&](int step, uint4 (&cq)[RB], uint32_t (&cd)[RB], uint4 (&pq)[RB], uint32_t (&pd)[RB]) {
    if (step >= n_steps) return;
    if (step + 2 < n_steps) load_step(step + 2, pq, pd);
    const int b = step / steps_per_batch;
    const int p = step - b * steps_per_batch;
    const bool tail = p == Qs;
    const int64_t row0 = r_begin + (int64_t)b * RB;
    const int rows_here = (int)(r_end - row0 < RB ? r_end - row0 : RB);
    const int chunk = tail ? tail_chunk : (p << 6) + lane;
    // rows with data in this step (uniform); idle tail lanes hold zero codes
    // and zero scales, so they add nothing
    const int nloads = __builtin_amdgcn_readfirstlane(tail ? RBt : rows_here);

    float S[RB][M];
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int m = 0; m < M; ++m) S[j][m] = 0.f;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      uint32_t xw[M][F::XDW];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4* src = reinterpret_cast<const uint4*>(xs + (m * MC + chunk) * CS + wi * F::XDW);
#pragma unroll
        for (int i = 0; i < F::XDW / 4; ++i) {
          const uint4 t = src[i];
          xw[m][4 * i] = t.x; xw[m][4 * i + 1] = t.y; xw[m][4 * i + 2] = t.z; xw[m][4 * i + 3] = t.w;
        }
      }
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (j < nloads) {
          const uint32_t w = wi == 0 ? cq[j].x : wi == 1 ? cq[j].y : wi == 2 ? cq[j].z : cq[j].w;
          if (FMT == kFmtPQ2) {
            const uint32_t e = w & 0x33333333u;         // codes 0,2,..,14 (one per nibble)
            const uint32_t o = (w >> 2) & 0x33333333u;  // codes 1,3,..,15
            f16x2 h[8];
            h[0] = codes2h<0>(e); h[1] = codes2h<0>(o);
            h[2] = codes2h<1>(e); h[3] = codes2h<1>(o);
            h[4] = codes2h<2>(e); h[5] = codes2h<2>(o);
            h[6] = codes2h<3>(e); h[7] = codes2h<3>(o);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
              for (int i = 0; i < 8; ++i) S[j][m] = dot2(h[i], xw[m][i], S[j][m]);
          } else {
            float v[4];
            v[0] = (float)(int8_t)(w);
            v[1] = (float)(int8_t)(w >> 8);
            v[2] = (float)(int8_t)(w >> 16);
            v[3] = (float)(int8_t)(w >> 24);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
              for (int i = 0; i < 4; ++i) S[j][m] = fmaf(v[i], __uint_as_float(xw[m][i]), S[j][m]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float X = F::FOLD ? xsum[m * MC + chunk] : 0.f;
      const float inv = F::FOLD ? xinv[m * MC + chunk] : 1.f;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (j < nloads) {
          const float t = F::FOLD ? (S[j][m] - X) : S[j][m];
          const float dj = F::FOLD ? f16_bits_to_f32(cd[j]) * inv : f16_bits_to_f32(cd[j]);
          if (tail)
            tacc[j][m] = fmaf(dj, t, tacc[j][m]);
          else
            acc[j][m] = fmaf(dj, t, acc[j][m]);
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
      if (Ts >= 2 && (Ts & (Ts - 1)) == 0 && Ts <= 32) {
        // tail partials: lane l of tail load j holds row G*j + l/Ts; sum each
        // aligned group of Ts lanes with DPP, then read the group totals
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          if (j < RBt) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const float t = group_sum_pow2(tacc[j][m], Ts);
              for (int g = 0; g < G; ++g) {
                const int r = G * j + g;
                const float tr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), g * Ts));
                if (r < rows_here) mine[m] = lane == r ? mine[m] + tr : mine[m];
              }
            }
          }
        }
      } else if (Ts) {
        // other tails: through the per-wave LDS scratch (LDS operations of a
        // wave complete in order; only compiler reordering must be stopped)
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
          for (int m = 0; m < M; ++m) scratch[(j * M + m) * 64 + lane] = tacc[j][m];
        __builtin_amdgcn_wave_barrier();
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
        __builtin_amdgcn_wave_barrier();
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
  };

  // three rotating register buffers: step s computes from buffer s % 3 and
  // prefetches step s + 2 into buffer (s + 2) % 3
  for (int step = 0; step < n_steps; step += 3) {
    body(step, q0, d0, q2, d2);
    body(step + 1, q1, d1, q0, d0);
    body(step + 2, q2, d2, q1, d1);
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
static constexpr int kLdsBudget = 120 * 1024;
static constexpr int kTargetWaves = 2048;  // 256 CUs x 4 SIMDs x 2

// LDS per workgroup: staged x' (+ per-chunk sum and range scale for PQ2_0)
// and, only when some K-slice has a tail step, the per-wave tail scratch.
static int64_t lds_bytes_for(int fmt, int64_t M, int n_groups, int S) {
  const int chunk_dw = fmt == kFmtPQ2 ? 32 : 16;
  const int chunks = 2 * ((n_groups + S - 1) / S);
  int64_t b = M * chunks * (chunk_dw + kPadDW) * 4;
  if (fmt == kFmtPQ2) b += 2 * M * chunks * 4;
  bool tail = false;
  for (int s = 0; s < S; ++s) {
    const int g0 = (int)((int64_t)s * n_groups / S), g1 = (int)((int64_t)(s + 1) * n_groups / S);
    tail = tail || ((2 * (g1 - g0)) & 63) != 0;
  }
  if (tail) b += (int64_t)kWaves * rows_per_batch(M) * M * 64 * 4;  // (used for odd tails only)
  return b;
}

GemvPlan plan_gemv(int fmt, int64_t M, int64_t N, int64_t K, int split_req) {
  GemvPlan p{};
  const int n_groups = (int)(K / group_of(fmt));
  int s_min = 1;
  while (s_min <= n_groups && lds_bytes_for(fmt, M, n_groups, s_min) > kLdsBudget) ++s_min;
  int S = split_req > 0 ? split_req : s_min;
  if (S > n_groups || S < 1 || lds_bytes_for(fmt, M, n_groups, S) > kLdsBudget) {
    p.split = -1;
    return p;
  }
  p.split = S;
  p.lds_bytes = (int)lds_bytes_for(fmt, M, n_groups, S);
  int64_t waves = kTargetWaves / S;
  if (waves < kWaves) waves = kWaves;
  int64_t rpw = (N + waves - 1) / waves;
  if (rpw < 1) rpw = 1;
  p.rows_per_wave = (int)rpw;
  int64_t w_needed = (N + rpw - 1) / rpw;
  p.grid_x = (int)((w_needed + kWaves - 1) / kWaves);
  return p;
}

// The rotation runs inside the GEMV prologue when every K-slice starts on an
// n-block boundary; otherwise a separate pre-pass writes x' to the workspace.
static bool rotation_fused(int fmt, int n_groups, int S, int block_len) {
  if (block_len <= 1) return true;
  const int g = group_of(fmt);
  for (int s = 0; s < S; ++s) {
    const int64_t k0 = (int64_t)s * n_groups / S * g;
    if (k0 % block_len) return false;
  }
  return (int64_t)n_groups * g % block_len == 0;
}

int64_t gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int block_len,
                             int split_req) {
  GemvPlan p = plan_gemv(fmt, M, N, K, split_req);
  if (p.split < 1) return -1;
  const int n_groups = (int)(K / group_of(fmt));
  int64_t b = 0;
  if (!rotation_fused(fmt, n_groups, p.split, block_len)) b += (M * K * 4 + 255) / 256 * 256;
  if (p.split > 1) b += (int64_t)p.split * M * N * 4;
  return b;
}

template <int FMT, int M>
static int launch_one(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  // more than 64 KiB of dynamic LDS needs the attribute; set once per
  // instantiation (thread-safe static initialisation)
  static const bool attr_ok =
      hipFuncSetAttribute((const void*)gemv_kernel<FMT, M>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) == hipSuccess;
  if (!attr_ok) return -1;
  dim3 grid(p.grid_x, p.split);
  gemv_kernel<FMT, M><<<grid, kThreads, p.lds_bytes, st>>>(a);
  return 0;
}

template <int FMT>
static int launch_fmt(int64_t M, const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  switch (M) {
    case 1: return launch_one<FMT, 1>(a, p, st);
    case 2: return launch_one<FMT, 2>(a, p, st);
    case 3: return launch_one<FMT, 3>(a, p, st);
    case 4: return launch_one<FMT, 4>(a, p, st);
    case 5: return launch_one<FMT, 5>(a, p, st);
    case 6: return launch_one<FMT, 6>(a, p, st);
    case 7: return launch_one<FMT, 7>(a, p, st);
    default: return launch_one<FMT, 8>(a, p, st);
  }
}

int launch_gemv(int fmt, const void* packed, int64_t N, int64_t K, const float* x, int64_t M,
                int block_len, const int8_t* signs, int split_req, float* y, void* ws,
                hipStream_t st) {
  GemvPlan p = plan_gemv(fmt, M, N, K, split_req);
  if (p.split < 1) return -2;
  const int n_groups = (int)(K / group_of(fmt));
  GemvArgs a;
  uint8_t* wsp = (uint8_t*)ws;
  if (rotation_fused(fmt, n_groups, p.split, block_len)) {
    a.x = x;
    a.signs = signs;
    int log2n = 0;
    while ((1 << log2n) < block_len) ++log2n;
    a.log2n = log2n;
    a.scale = block_len > 1 ? (float)(1.0 / __builtin_sqrt((double)block_len)) : 1.0f;
  } else {
    float* xprime = (float*)wsp;
    if (launch_hadamard(x, 0, xprime, 0, M, K, block_len, signs, st)) return -1;
    wsp += (M * K * 4 + 255) / 256 * 256;
    a.x = xprime;
    a.signs = nullptr;
    a.log2n = 0;
    a.scale = 1.0f;
  }
  PlanarView pv = planar_view(fmt, N, K, const_cast<void*>(packed));
  a.qs = pv.qs;
  a.dpl = (const uint16_t*)pv.d;
  a.N = N;
  a.K = K;
  a.row_bytes = (int)pv.row_bytes;
  a.d_per_row = (int)pv.d_per_row;
  a.n_groups = n_groups;
  a.split = p.split;
  a.rows_per_wave = p.rows_per_wave;
  a.max_slice_chunks = 2 * ((n_groups + p.split - 1) / p.split);
  float* part = p.split > 1 ? (float*)wsp : nullptr;
  a.out = p.split > 1 ? part : y;
  const int rc = fmt == kFmtPQ2 ? launch_fmt<kFmtPQ2>(M, a, p, st) : launch_fmt<kFmtQ8>(M, a, p, st);
  if (rc || hipGetLastError() != hipSuccess) return -1;
  if (p.split > 1) {
    int64_t n = M * N;
    splitk_reduce_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(part, y, n, p.split);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace kq
