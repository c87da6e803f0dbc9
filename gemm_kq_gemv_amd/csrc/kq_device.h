// kq_device.h -- device helpers shared by the HIP kernels of libkq (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// IEEE binary16 <-> binary32 through the hardware converters (round to
// nearest even, subnormals kept).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// bfloat16 <-> binary32 (round to nearest even on the way down).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Two 2-bit codes of one byte of a nibble-spread word -> two floats.
// `spread` holds one code in the low two bits of each nibble (upper two bits
// zero), which is an E2M1 (fp4) value c/2; with scale 2.0 the converter
// returns the code itself, exactly.  SEL picks the byte (0..3): low nibble
// -> .x, high nibble -> .y.
template <int SEL>
__device__ __forceinline__ f32x2 codes2(uint32_t spread) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(spread, 2.0f, SEL);
}

// Sum over the 64 lanes of a wave; every lane receives the total.
// Four DPP stages reduce within each row of 16 lanes, the four row sums are
// then read out and added in a fixed order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
  // xor 1, xor 2 (quad permutes), mirror within 8, mirror within 16
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Sum over each aligned group of n lanes (n in {2, 4, 8, 16, 32}); every lane
// of a group receives its group's total.
__device__ __forceinline__ float group_sum_pow2(float v, int n) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  if (n >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  if (n >= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  if (n >= 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  if (n >= 32) v += __shfl_xor(v, 16);
  return v;
}

// Raw buffer access (gfx9 buffer resource, stride 0): loads whose byte offset
// lies outside [0, num_bytes) return zero instead of touching memory.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
// Code plane tiling: the 32 code bytes of block b of row n live in tile
// (n / 16, b) -- 16 rows x 32 bytes, row n % 16 at byte 32 * (n % 16) -- and
// tile (t, b) starts at byte 512 * (t * nb + b).  A pair of blocks of a
// 16-row block is then 1 KiB of contiguous memory.  Word index of 32-bit word
// wr (of K/16 or K/4 per row) of row n, for nb blocks per row:
__host__ __device__ __forceinline__ int64_t tiled_word(int64_t n, int64_t wr, int64_t nb) {
  return (((n >> 4) * nb + (wr >> 3)) << 7) + ((n & 15) << 3) + (wr & 7);
}
// PQ2_0 code words in the code plane.  The block's word i (its code bytes
// 4i..4i+3, little-endian) holds codes 16i + j at bits 2j (low bit b0) and
// 2j + 1 (high bit b1).  The stored word keeps every b0 in place and rotates
// the b1 bits up by two: b1 of code j sits at bit (2j + 3) mod 32.  Then
// codes 2i have their bits at 4i and 4i + 3, codes 2i + 1 at 4i + 2 and
// 4i + 5, exactly the sign and mantissa bits of fp4 nibble i once the word
// (or, for the odd codes, the word rotated down by two) is complemented and
// masked: two and three instructions for the GEMV's operands.
__host__ __device__ __forceinline__ uint32_t pq2_store_word(uint32_t w) {
  const uint32_t hi = w & 0xAAAAAAAAu;
  return (w & 0x55555555u) | (hi << 2) | (hi >> 30);
}
__host__ __device__ __forceinline__ uint32_t pq2_load_word(uint32_t s) {
  const uint32_t hi = s & 0xAAAAAAAAu;
  return (s & 0x55555555u) | (hi >> 2) | (hi << 30);
}
// Scale plane tiling: the fp16 scale of block b of row n lives in chunk
// (n / 16, b / 8) -- 16 rows x 8 blocks, row n % 16 at byte 16 * (n % 16),
// block b % 8 at byte 2 * (b % 8) within it -- and chunk (t, c) starts at
// byte 256 * (t * C + c), C = ceil(nb / 8).  The 8 scales of a row within a
// chunk are 16 contiguous bytes, and a 16-row block's scales for 8 blocks one
// 256-byte run.  Index in 16-bit units:
__host__ __device__ __forceinline__ int64_t tiled_scale(int64_t n, int64_t b, int64_t C) {
  return (((n >> 4) * C + (b >> 3)) << 7) + ((n & 15) << 3) + (b & 7);
}
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;  // an offset past any range used here
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 buffer_load_16B(BufRsrc r, uint32_t off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Streamed weights: the non-temporal hint (cache-policy bit 1 on gfx950)
// keeps data that is read once from displacing reused lines in the caches.
__device__ __forceinline__ uint4 buffer_load_16B_stream(BufRsrc r, uint32_t off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t buffer_load_2B(BufRsrc r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

}  // namespace kq
