// pack.hip -- PQ2_0 / Q8_0 quantizers and dequantizers (planar layout), and
// the PTQ1_0 -> PQ2_0 transcode.
//
// PQ2_0 (Bonsai 2 27B ternary g128 page, sec. 3.1): per 128-group
// d = max|w| stored as fp16, q = round(w/d) + 1, element j in byte j/4 at bit
// offset 2(j%4).  Q8_0 (Kipp architecture page, "Weight quantization"):
// per 32-group the scale max|w|/127 stored as fp16, q = round(w/scale)
// against the fp16-rounded scale.  Rounding is half away from zero, the
// division is the IEEE one, and an all-zero group keeps d = 0 with the
// neutral code (1 for PQ2_0, 0 for Q8_0).
//
// PQ2_0 words are stored with their high code bits rotated (pq2_store_word).
//
// Launch shape: one thread per 32-bit code word, in row-major order over the
// rows padded to whole 16-row tiles.  For PQ2_0 a word holds 16 codes and 8
// consecutive threads cover one 128-group; for Q8_0 a word holds 4 int8 and 8
// threads cover one 32-group.  The group max is reduced across those 8 lanes
// with xor shuffles, so one pass reads W once with coalesced 64/16-byte loads;
// each group's 8 words land as 32 contiguous bytes of its tile, and padding
// rows are written as zeros.  The group's first thread writes its scale into
// the tiled scale plane (zero for padding rows); the thread of a row's last
// block also zeroes the unused block slots of that row's last chunk.
#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

// scale of the group whose first code word is g (words_per_row = 8 nb); the
// last block of a row also clears the padding slots of its chunk
__device__ __forceinline__ void store_scale(uint16_t* dplane, int64_t g, int64_t words_per_row, int64_t C,
                                            uint16_t d16) {
  const int64_t n = g / words_per_row, b = (g % words_per_row) >> 3, nb = words_per_row >> 3;
  dplane[tiled_scale(n, b, C)] = d16;
  if (b == nb - 1)
    for (int64_t p = nb; p < 8 * C; ++p) dplane[tiled_scale(n, p, C)] = 0;
}

__device__ __forceinline__ float group8_max(float a) {
  // the 8 lanes of a group are aligned to 8 within the wave
  a = fmaxf(a, __shfl_xor(a, 1, 8));
  a = fmaxf(a, __shfl_xor(a, 2, 8));
  a = fmaxf(a, __shfl_xor(a, 4, 8));
  return a;
}

__global__ __launch_bounds__(256) void pack_pq2_kernel(
    const float* __restrict__ W, uint32_t* __restrict__ qs, uint16_t* __restrict__ dplane,
    int64_t n_words, int64_t live_words, int64_t words_per_row, int64_t C) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool in_plane = g < n_words;
  bool live = g < live_words;
  float w[16];
  if (live) {
    const float4* src = reinterpret_cast<const float4*>(W) + g * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 v = src[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(w[i]));
  amax = group8_max(amax);
  uint16_t d16 = f32_to_f16_bits(amax);
  float dF = f16_bits_to_f32(d16);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int q = 1;
    if (dF != 0.f) {
      q = (int)roundf(w[j] / dF) + 1;  // IEEE division, ties away from zero
      q = q < 0 ? 0 : (q > 2 ? 2 : q);
    }
    word |= (uint32_t)q << (2 * j);
  }
  if (in_plane) {
    qs[tiled_word(g / words_per_row, g % words_per_row, words_per_row >> 3)] = live ? pq2_store_word(word) : 0u;
    if ((g & 7) == 0) store_scale(dplane, g, words_per_row, C, live ? d16 : (uint16_t)0);
  }
}

__global__ __launch_bounds__(256) void pack_q8_kernel(
    const float* __restrict__ W, uint32_t* __restrict__ qs, uint16_t* __restrict__ dplane,
    int64_t n_words, int64_t live_words, int64_t words_per_row, int64_t C) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool in_plane = g < n_words;
  bool live = g < live_words;
  float4 v = live ? reinterpret_cast<const float4*>(W)[g] : make_float4(0.f, 0.f, 0.f, 0.f);
  float w[4] = {v.x, v.y, v.z, v.w};
  float amax = fmaxf(fmaxf(fabsf(w[0]), fabsf(w[1])), fmaxf(fabsf(w[2]), fabsf(w[3])));
  amax = group8_max(amax);
  float d32 = amax / 127.0f;  // IEEE division
  uint16_t d16 = f32_to_f16_bits(d32);
  float dF = f16_bits_to_f32(d16);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int q = 0;
    if (dF != 0.f) {
      q = (int)roundf(w[j] / dF);
      q = q < -127 ? -127 : (q > 127 ? 127 : q);
    }
    word |= ((uint32_t)q & 0xFFu) << (8 * j);
  }
  if (in_plane) {
    qs[tiled_word(g / words_per_row, g % words_per_row, words_per_row >> 3)] = live ? word : 0u;
    if ((g & 7) == 0) store_scale(dplane, g, words_per_row, C, live ? d16 : (uint16_t)0);
  }
}

// Dequantize: one thread per 32-bit code word of the N real rows (row-major).
__global__ __launch_bounds__(256) void unpack_pq2_kernel(
    const uint32_t* __restrict__ qs, const uint16_t* __restrict__ dplane,
    float* __restrict__ W, int64_t n_words, int64_t words_per_row, int64_t C) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_words) return;
  uint32_t word = pq2_load_word(qs[tiled_word(g / words_per_row, g % words_per_row, words_per_row >> 3)]);
  float d = f16_bits_to_f32(dplane[tiled_scale(g / words_per_row, (g % words_per_row) >> 3, C)]);
  float4* dst = reinterpret_cast<float4*>(W) + g * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (float)((int)((word >> (2 * (4 * i + j))) & 3u) - 1) * d;
    dst[i] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

__global__ __launch_bounds__(256) void unpack_q8_kernel(
    const uint32_t* __restrict__ qs, const uint16_t* __restrict__ dplane,
    float* __restrict__ W, int64_t n_words, int64_t words_per_row, int64_t C) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_words) return;
  uint32_t word = qs[tiled_word(g / words_per_row, g % words_per_row, words_per_row >> 3)];
  float d = f16_bits_to_f32(dplane[tiled_scale(g / words_per_row, (g % words_per_row) >> 3, C)]);
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = d * (float)(int8_t)(word >> (8 * j));
  reinterpret_cast<float4*>(W)[g] = make_float4(v[0], v[1], v[2], v[3]);
}

// PTQ1_0 -> PQ2_0 (Bonsai page, sec. 3.2: the two packs carry the same trits
// and scales, so PTQ1_0 is a download format that is turned into PQ2_0 words
// at load time).  A PTQ1_0 block is 24 bytes of five base-3 digits and 2 of
// four, then the fp16 scale (28 bytes).  Element e of a block:
//   e <  80: digit e / 16 of byte e % 16
//   e < 120: digit (e - 80) / 8 of byte 16 + (e - 80) % 8
//   else:    digit (e - 120) / 2 of byte 24 + (e - 120) % 2
// and digit n of byte q is ((q * 3^n) mod 256) * 3 / 256 (0, 1 or 2 for any
// byte).  Same launch shape as the packers: one thread per 32-bit PQ2_0 code
// word (16 elements) of the padded plane; the 8 threads of a group read the
// same 28 bytes as seven aligned words.
__device__ __forceinline__ uint32_t ptq1_digit(uint32_t q, int n) {
  const uint32_t p3 = n == 0 ? 1u : n == 1 ? 3u : n == 2 ? 9u : n == 3 ? 27u : 81u;
  return (((q * p3) & 0xFFu) * 3u) >> 8;
}

__global__ __launch_bounds__(256) void transcode_ptq1_kernel(
    const uint32_t* __restrict__ src, uint32_t* __restrict__ qs, uint16_t* __restrict__ dplane,
    int64_t n_words, int64_t live_words, int64_t words_per_row, int64_t C) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_words) return;
  const bool live = g < live_words;
  const int64_t blk = g >> 3;  // block index, row-major (live words only)
  const int i = (int)(g & 7);  // code word of the block: elements 16 i .. 16 i + 15
  uint32_t t[7] = {0u, 0u, 0u, 0u, 0u, 0u, 0u};
  if (live) {
#pragma unroll
    for (int k = 0; k < 7; ++k) t[k] = src[blk * 7 + k];
  }
  auto byte_at = [&](int k) { return (t[k >> 2] >> (8 * (k & 3))) & 0xFFu; };
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = 16 * i + j;
    const int byte = e < 80 ? e % 16 : e < 120 ? 16 + (e - 80) % 8 : 24 + (e - 120) % 2;
    const int n = e < 80 ? e / 16 : e < 120 ? (e - 80) / 8 : (e - 120) / 2;
    word |= ptq1_digit(byte_at(byte), n) << (2 * j);
  }
  qs[tiled_word(g / words_per_row, g % words_per_row, words_per_row >> 3)] = live ? pq2_store_word(word) : 0u;
  if (i == 0)
    store_scale(dplane, g, words_per_row, C, live ? (uint16_t)(byte_at(26) | (byte_at(27) << 8)) : (uint16_t)0);
}

static int blocks_for(int64_t n) { return (int)((n + 255) / 256); }

int launch_pack(int fmt, const float* W, int64_t N, int64_t K, void* packed,
                hipStream_t st) {
  PlanarView pv = planar_view(fmt, N, K, packed);
  const int64_t n_words = pv.qs_bytes / 4, wpr = pv.row_bytes / 4, live = N * wpr;
  if (n_words == 0) return 0;
  if (fmt == 1)
    pack_pq2_kernel<<<blocks_for(n_words), 256, 0, st>>>(W, (uint32_t*)pv.qs, (uint16_t*)pv.d, n_words, live, wpr, pv.d_chunks);
  else
    pack_q8_kernel<<<blocks_for(n_words), 256, 0, st>>>(W, (uint32_t*)pv.qs, (uint16_t*)pv.d, n_words, live, wpr, pv.d_chunks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_transcode_ptq1(const void* ptq1, int64_t N, int64_t K, void* packed, hipStream_t st) {
  PlanarView pv = planar_view(kFmtPQ2, N, K, packed);
  const int64_t n_words = pv.qs_bytes / 4, wpr = pv.row_bytes / 4, live = N * wpr;
  if (n_words == 0) return 0;
  transcode_ptq1_kernel<<<blocks_for(n_words), 256, 0, st>>>((const uint32_t*)ptq1, (uint32_t*)pv.qs,
                                                             (uint16_t*)pv.d, n_words, live, wpr,
                                                             pv.d_chunks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_unpack(int fmt, const void* packed, int64_t N, int64_t K, float* W,
                  hipStream_t st) {
  PlanarView pv = planar_view(fmt, N, K, const_cast<void*>(packed));
  const int64_t wpr = pv.row_bytes / 4, n_words = N * wpr;
  if (n_words == 0) return 0;
  if (fmt == 1)
    unpack_pq2_kernel<<<blocks_for(n_words), 256, 0, st>>>((const uint32_t*)pv.qs, (const uint16_t*)pv.d, W, n_words, wpr, pv.d_chunks);
  else
    unpack_q8_kernel<<<blocks_for(n_words), 256, 0, st>>>((const uint32_t*)pv.qs, (const uint16_t*)pv.d, W, n_words, wpr, pv.d_chunks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kq
