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

}  // namespace kq
