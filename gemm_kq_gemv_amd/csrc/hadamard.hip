// hadamard.hip -- blockwise Walsh-Hadamard pre-pass.
//
// Bonsai 2 27B ternary g128 page, sec. 4.1-4.2: x' = (1/sqrt(n)) H_n (s (.) x)
// for each n-block of a row (block-diagonal along K), H_n in Sylvester
// natural order, the sign flip applied before the transform.
//
// Layout on gfx950: each thread owns 16 consecutive elements, so an n-block
// (n <= 1024) spans n/16 <= 64 aligned lanes of one wave.  The butterflies
// with stride < 16 run in registers; the wider ones pair lanes with xor
// shuffles (lane distance 1..32).  No LDS and no barrier are needed: a
// 1024-point block is exactly one wave.  Arithmetic is fp32 (one rounding to
// bf16 at the store for bf16 output), and the 1/sqrt(n) factor is applied
// once at the end.
#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void hadamard_kernel(
    const void* __restrict__ x, void* __restrict__ xr, const int8_t* __restrict__ signs,
    int64_t n_groups, int64_t K, int log2n, float scale) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool live = g < n_groups;
  float v[16];
  if (live) {
    if (IN_BF16) {
      const uint4* src = reinterpret_cast<const uint4*>(x) + g * 2;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint4 u = src[i];
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
          v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
        }
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(x) + g * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    }
    if (signs) {
      int64_t k0 = (g * 16) % K;
      uint4 s = *reinterpret_cast<const uint4*>(signs + k0);
      uint32_t sw[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        uint32_t neg = (sw[j >> 2] >> (8 * (j & 3) + 7)) & 1u;  // sign bit of the int8
        v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (neg << 31));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = 0.f;
  }

  // in-register butterflies, strides 1, 2, 4, 8 (as far as the block reaches)
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < log2n) {
      const int h = 1 << s;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if ((i & h) == 0) {
          float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
        }
      }
    }
  }
  // cross-lane butterflies, lane distance 1 .. 32
  const int lane = lane_id();
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    if (s + 4 < log2n) {
      const int h = 1 << s;
      const bool upper = (lane & h) != 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = __shfl_xor(v[i], h);
        v[i] = upper ? (p - v[i]) : (v[i] + p);
      }
    }
  }

  if (!live) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] *= scale;
  if (OUT_BF16) {
    uint4* dst = reinterpret_cast<uint4*>(xr) + g * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint4 u;
      u.x = pack_bf16x2(v[8 * i + 0], v[8 * i + 1]);
      u.y = pack_bf16x2(v[8 * i + 2], v[8 * i + 3]);
      u.z = pack_bf16x2(v[8 * i + 4], v[8 * i + 5]);
      u.w = pack_bf16x2(v[8 * i + 6], v[8 * i + 7]);
      dst[i] = u;
    }
  } else {
    float4* dst = reinterpret_cast<float4*>(xr) + g * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

int launch_hadamard(const void* x, int x_bf16, void* xr, int xr_bf16, int64_t M, int64_t K,
                    int n, const int8_t* signs, hipStream_t st) {
  int64_t n_groups = M * K / 16;
  if (n_groups == 0) return 0;
  int log2n = 0;
  while ((1 << log2n) < n) ++log2n;
  float scale = (float)(1.0 / __builtin_sqrt((double)n));
  int blocks = (int)((n_groups + 255) / 256);
  if (x_bf16 && xr_bf16)
    hadamard_kernel<true, true><<<blocks, 256, 0, st>>>(x, xr, signs, n_groups, K, log2n, scale);
  else if (x_bf16)
    hadamard_kernel<true, false><<<blocks, 256, 0, st>>>(x, xr, signs, n_groups, K, log2n, scale);
  else if (xr_bf16)
    hadamard_kernel<false, true><<<blocks, 256, 0, st>>>(x, xr, signs, n_groups, K, log2n, scale);
  else
    hadamard_kernel<false, false><<<blocks, 256, 0, st>>>(x, xr, signs, n_groups, K, log2n, scale);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kq
