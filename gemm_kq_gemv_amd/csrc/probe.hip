// probe.hip -- measurement instruments (include/kq_probe.h): a streaming
// read-reduce, the reachable HBM read rate on this GPU; a matrix-core issue
// loop, the reachable bf16 MFMA rate; and the entry point of the GEMV's
// loads-only twin (its kernel sits beside the GEMV kernels, so that both use
// the same row-block load code).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kq_probe.h"
#include "kq_device.h"
#include "kq_launch.h"

namespace kq {

// 16-byte non-temporal loads, U in flight per thread, XOR-reduced.
// layout 0: grid-stride over the 16-byte units; 1: workgroup b reads the
// b-th of gridDim.x contiguous chunks.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int LAYOUT>
__global__ __launch_bounds__(1024) void probe_read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                          uint32_t* sink) {
  constexpr int U = 4;
  uint64_t b0 = 0, b1 = n16, i, st;
  if constexpr (LAYOUT == 0) {
    i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    st = (uint64_t)gridDim.x * blockDim.x;
  } else {
    const uint64_t C = (n16 + gridDim.x - 1) / gridDim.x;
    b0 = (uint64_t)blockIdx.x * C;
    b1 = b0 + C < n16 ? b0 + C : n16;
    i = b0 + threadIdx.x;
    st = blockDim.x;
  }
  uint32_t acc = 0;
  for (; i + (U - 1) * st < b1; i += U * st) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * st);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += st) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

int launch_probe_read(const void* buf, size_t bytes, int layout, int grid, int block,
                      uint32_t* sink, hipStream_t st) {
  const u32x4* p = (const u32x4*)buf;
  const uint64_t n16 = bytes / 16;
  if (layout == 0)
    hipLaunchKernelGGL(probe_read_kernel<0>, dim3(grid), dim3(block), 0, st, p, n16, sink);
  else
    hipLaunchKernelGGL(probe_read_kernel<1>, dim3(grid), dim3(block), 0, st, p, n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Matrix-core issue ceiling: every wave runs `iters` rounds of kChains
// independent v_mfma_f32_16x16x32_bf16 (the prefill GEMM's instruction) on
// operands held in registers, and only then sums its accumulators.  The
// operand values are small multiples of 1/16, so the sums stay finite.
constexpr int kMfmaChains = 16;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(1024) void probe_mfma_kernel(int iters, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.0625f * (float)((lane + i) & 3));
    b[i] = (__bf16)(0.0625f * (float)((lane + 2 * i) & 3));
  }
  f32x4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  if (__float_as_uint(s) == 0x9E3779B9u) sink[0] = __float_as_uint(s);
}

int launch_probe_mfma(int iters, int grid, int block, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(block), 0, st, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kq

namespace {
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
}  // namespace

extern "C" {

kq_status kq_probe_read(const void* buf, size_t bytes, int32_t layout, int32_t grid, int32_t block,
                        uint32_t* sink, void* stream) {
  if (!buf || !sink || (layout != 0 && layout != 1)) return KQ_EINVAL;
  if (grid < 1 || grid > 65536 || block < 64 || block > 1024 || block % 64 || bytes < 16 ||
      bytes % 16)
    return KQ_ESHAPE;
  if (!aligned16(buf) || !aligned16(sink)) return KQ_EALIGN;
  return kq::launch_probe_read(buf, bytes, layout, grid, block, sink, (hipStream_t)stream) == 0
             ? KQ_OK
             : KQ_EDEVICE;
}

kq_status kq_probe_mfma(int32_t iters, int32_t grid, int32_t block, uint32_t* sink, void* stream) {
  if (!sink) return KQ_EINVAL;
  if (iters < 1 || iters > (1 << 20) || grid < 1 || grid > 65536 || block < 64 || block > 1024 ||
      block % 64)
    return KQ_ESHAPE;
  if (!aligned16(sink)) return KQ_EALIGN;
  return kq::launch_probe_mfma(iters, grid, block, sink, (hipStream_t)stream) == 0 ? KQ_OK
                                                                                   : KQ_EDEVICE;
}

kq_status kq_probe_gemv_loads(kq_format fmt, const void* packed, int64_t N, int64_t K,
                              const float* x, int64_t M, int32_t block_len, int32_t split_k,
                              uint32_t* sink, void* stream) {
  // the argument contract of kq_gemv (without signs, output and workspace)
  if ((fmt != KQ_FMT_PQ2_0 && fmt != KQ_FMT_Q8_0) || !packed || !x || !sink) return KQ_EINVAL;
  if (N < 0 || K < 0 || M < 0) return KQ_EINVAL;
  const int64_t g = fmt == KQ_FMT_PQ2_0 ? 128 : 32;
  const bool bl_ok = block_len == 0 || (block_len >= 1 && block_len <= 1024 && !(block_len & (block_len - 1)));
  if (N < 1 || K < g || K % g || N > (int64_t(1) << 40) / K || M < 1 || M > 8 || !bl_ok ||
      (block_len > 0 && K % block_len) || split_k < 0 || split_k > K / g)
    return KQ_ESHAPE;
  if (!aligned16(packed) || !aligned16(x) || !aligned16(sink)) return KQ_EALIGN;
  const int rc = kq::launch_gemv_loads_twin(fmt, packed, N, K, x, M, block_len, split_k, sink,
                                            (hipStream_t)stream);
  return rc == 0 ? KQ_OK : rc == -2 ? KQ_EUNSUPPORTED : KQ_EDEVICE;
}

}  // extern "C"
