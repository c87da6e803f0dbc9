// api.hip -- the extern "C" entry points declared in include/kq.h.
// Validation happens here, before anything is enqueued; the kernels assume
// the shapes they receive are valid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/kq.h"
#include "kq_launch.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool fmt_ok(kq_format f) { return f == KQ_FMT_PQ2_0 || f == KQ_FMT_Q8_0; }
bool dtype_ok(kq_dtype d) { return d == KQ_F32 || d == KQ_BF16; }
bool block_len_ok(int32_t n) { return n == 0 || (n >= 1 && n <= 1024 && (n & (n - 1)) == 0); }
bool shape_ok(kq_format f, int64_t N, int64_t K) {
  const int g = f == KQ_FMT_PQ2_0 ? 128 : 32;
  return N >= 1 && K >= g && K % g == 0 && N <= (int64_t(1) << 40) / K;
}
hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Scratch memory of kq_gemv_noalloc (the split-K partials), for callers that
// cannot allocate: one static array per GPU, alive until the process ends.
// Host code uses its per-device address from hipGetSymbolAddress, never the
// array's name (a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];  // per device, set on its first call

// Address of the current device's scratch array, resolved once per device with
// that device current; NULL if the runtime cannot tell it.
void* current_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}
kq_status launched(int rc) { return rc == 0 ? KQ_OK : KQ_EDEVICE; }

}  // namespace

extern "C" {

const char* kq_status_string(kq_status s) {
  switch (s) {
    case KQ_OK: return "KQ_OK";
    case KQ_EINVAL: return "KQ_EINVAL: null pointer, unknown enum or negative size";
    case KQ_ESHAPE: return "KQ_ESHAPE: shape, block_len or split_k out of contract";
    case KQ_EALIGN: return "KQ_EALIGN: pointer not 16-byte aligned";
    case KQ_EWORKSPACE: return "KQ_EWORKSPACE: workspace missing or too small";
    case KQ_EUNSUPPORTED: return "KQ_EUNSUPPORTED: unsupported combination";
    case KQ_EDEVICE: return "KQ_EDEVICE: the HIP runtime rejected a launch";
  }
  return "unknown kq_status";
}

size_t kq_packed_bytes(kq_format fmt, int64_t N, int64_t K) {
  if (!fmt_ok(fmt) || !shape_ok(fmt, N, K)) return 0;
  return (size_t)kq::planar_view(fmt, N, K, nullptr).total_bytes;
}

static kq_status check_pack(kq_format fmt, const void* W, int64_t N, int64_t K, const void* out) {
  if (!W || !out) return KQ_EINVAL;
  if (N < 0 || K < 0) return KQ_EINVAL;
  if (!shape_ok(fmt, N, K)) return KQ_ESHAPE;
  if (!aligned16(W) || !aligned16(out)) return KQ_EALIGN;
  return KQ_OK;
}

kq_status kq_pack_pq2(const float* W, int64_t N, int64_t K, void* packed, void* stream) {
  kq_status st = check_pack(KQ_FMT_PQ2_0, W, N, K, packed);
  if (st != KQ_OK) return st;
  return launched(kq::launch_pack(kq::kFmtPQ2, W, N, K, packed, as_stream(stream)));
}

kq_status kq_pack_q8(const float* W, int64_t N, int64_t K, void* packed, void* stream) {
  kq_status st = check_pack(KQ_FMT_Q8_0, W, N, K, packed);
  if (st != KQ_OK) return st;
  return launched(kq::launch_pack(kq::kFmtQ8, W, N, K, packed, as_stream(stream)));
}

kq_status kq_transcode_ptq1(const void* ptq1, int64_t N, int64_t K, void* packed, void* stream) {
  kq_status st = check_pack(KQ_FMT_PQ2_0, ptq1, N, K, packed);
  if (st != KQ_OK) return st;
  return launched(kq::launch_transcode_ptq1(ptq1, N, K, packed, as_stream(stream)));
}

kq_status kq_unpack(kq_format fmt, const void* packed, int64_t N, int64_t K, float* W_out,
                    void* stream) {
  if (!fmt_ok(fmt)) return KQ_EINVAL;
  kq_status st = check_pack(fmt, packed, N, K, W_out);
  if (st != KQ_OK) return st;
  return launched(kq::launch_unpack(fmt, packed, N, K, W_out, as_stream(stream)));
}

kq_status kq_hadamard_blocks(const void* x, kq_dtype x_dt, void* xr, kq_dtype xr_dt, int64_t M,
                             int64_t K, int32_t block_len, const int8_t* signs, void* stream) {
  if (!x || !xr || !dtype_ok(x_dt) || !dtype_ok(xr_dt)) return KQ_EINVAL;
  if (M < 0 || K < 0) return KQ_EINVAL;
  if (M < 1 || K < 16 || K % 16 || block_len < 1 || !block_len_ok(block_len) ||
      K % block_len || M > (int64_t(1) << 40) / K)
    return KQ_ESHAPE;
  if (!aligned16(x) || !aligned16(xr) || (signs && !aligned16(signs))) return KQ_EALIGN;
  return launched(kq::launch_hadamard(x, x_dt == KQ_BF16, xr, xr_dt == KQ_BF16, M, K, block_len,
                                      signs, as_stream(stream)));
}

size_t kq_workspace_bytes(int32_t op, kq_format fmt, int64_t M, int64_t N, int64_t K,
                          int32_t block_len, int32_t split_k) {
  if (!fmt_ok(fmt) || !shape_ok(fmt, N, K) || M < 1 || !block_len_ok(block_len)) return 0;
  if (op == 0) {
    if (M > 8 || split_k < 0) return 0;
    int64_t b = kq::gemv_workspace_bytes(fmt, M, N, K, block_len, split_k);
    return b < 0 ? 0 : (size_t)b;
  }
  if (op == 1) return (size_t)kq::gemm_workspace_bytes(fmt, M, N, K, block_len, 1, nullptr);
  return 0;
}

kq_status kq_gemv(kq_format fmt, const void* packed, int64_t N, int64_t K, const float* x,
                  int64_t M, int32_t block_len, const int8_t* signs, int32_t split_k, float* y,
                  void* workspace, size_t ws_bytes, void* stream) {
  if (!fmt_ok(fmt) || !packed || !x || !y) return KQ_EINVAL;
  if (N < 0 || K < 0 || M < 0) return KQ_EINVAL;
  if (!shape_ok(fmt, N, K) || M < 1 || M > 8 || !block_len_ok(block_len) ||
      (block_len > 0 && K % block_len) || split_k < 0)
    return KQ_ESHAPE;
  if (split_k > K / kq::group_of(fmt)) return KQ_ESHAPE;
  if (!aligned16(packed) || !aligned16(x) || !aligned16(y) || (signs && !aligned16(signs)) ||
      (workspace && !aligned16(workspace)))
    return KQ_EALIGN;
  kq::GemvPlan plan = kq::plan_gemv(fmt, M, N, K, block_len, split_k);
  if (plan.split < 1) return KQ_EUNSUPPORTED;  // no split fits the LDS or buffer-range limits
  const int64_t need = kq::gemv_workspace_bytes(fmt, M, N, K, block_len, split_k);
  if (need > 0 && (!workspace || (int64_t)ws_bytes < need)) return KQ_EWORKSPACE;
  const int rc = kq::launch_gemv(fmt, packed, N, K, x, M, block_len, signs, split_k, y, workspace,
                                 as_stream(stream));
  return rc == -2 ? KQ_EUNSUPPORTED : launched(rc);
}

kq_status kq_gemv_noalloc(kq_format fmt, const void* packed, int64_t N, int64_t K,
                          const float* x, int64_t M, int32_t block_len, const int8_t* signs,
                          int32_t split_k, float* y, void* stream) {
  if (!fmt_ok(fmt) || !packed || !x || !y) return KQ_EINVAL;
  if (N < 0 || K < 0 || M < 0) return KQ_EINVAL;
  if (!shape_ok(fmt, N, K) || M < 1 || M > 8 || !block_len_ok(block_len) ||
      (block_len > 0 && K % block_len) || split_k < 0)
    return KQ_ESHAPE;
  if (split_k > K / kq::group_of(fmt)) return KQ_ESHAPE;
  if (!aligned16(packed) || !aligned16(x) || !aligned16(y) || (signs && !aligned16(signs)))
    return KQ_EALIGN;
  kq::GemvPlan plan = kq::plan_gemv(fmt, M, N, K, block_len, split_k);
  if (plan.split < 1) return KQ_EUNSUPPORTED;
  const int64_t need = kq::gemv_workspace_bytes(fmt, M, N, K, block_len, split_k);
  if (need > (int64_t)kScratchBytes) return KQ_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0 && !(ws = current_scratch())) return KQ_EDEVICE;
  const int rc = kq::launch_gemv(fmt, packed, N, K, x, M, block_len, signs, split_k, y, ws,
                                 as_stream(stream));
  return rc == -2 ? KQ_EUNSUPPORTED : launched(rc);
}

kq_status kq_gemv_multi(kq_format fmt, int32_t nsets, const void* const* packed, const int64_t* N,
                        int64_t K, const float* x, int64_t M, int32_t block_len,
                        const int8_t* signs, float* const* y, void* stream) {
  if (!fmt_ok(fmt) || !packed || !N || !x || !y) return KQ_EINVAL;
  if (nsets < 1 || nsets > kq::kMaxSets) return KQ_ESHAPE;
  if (K < 0 || M < 0) return KQ_EINVAL;
  for (int s = 0; s < nsets; ++s) {
    if (!packed[s] || !y[s]) return KQ_EINVAL;
    if (N[s] < 0) return KQ_EINVAL;
  }
  for (int s = 0; s < nsets; ++s)
    if (!shape_ok(fmt, N[s], K)) return KQ_ESHAPE;
  if (M < 1 || M > 8 || !block_len_ok(block_len) || (block_len > 0 && K % block_len))
    return KQ_ESHAPE;
  if (!aligned16(x) || (signs && !aligned16(signs))) return KQ_EALIGN;
  for (int s = 0; s < nsets; ++s)
    if (!aligned16(packed[s]) || !aligned16(y[s])) return KQ_EALIGN;
  if (kq::check_gemv_multi(fmt, nsets, N, K, M, block_len)) return KQ_EUNSUPPORTED;
  const int rc = kq::launch_gemv_multi(fmt, nsets, packed, N, K, x, M, block_len, signs, y,
                                       as_stream(stream));
  return rc == -2 ? KQ_EUNSUPPORTED : launched(rc);
}

kq_status kq_gemm(kq_format fmt, const void* packed, int64_t N, int64_t K, const void* x,
                  kq_dtype x_dt, int64_t M, int32_t block_len, const int8_t* signs, float* y,
                  void* workspace, size_t ws_bytes, void* stream) {
  if (!fmt_ok(fmt) || !dtype_ok(x_dt) || !packed || !x || !y) return KQ_EINVAL;
  if (N < 0 || K < 0 || M < 0) return KQ_EINVAL;
  if (!shape_ok(fmt, N, K) || M < 1 || M > (int64_t(1) << 40) / K || !block_len_ok(block_len) ||
      (block_len > 0 && K % block_len))
    return KQ_ESHAPE;
  if (!aligned16(packed) || !aligned16(x) || !aligned16(y) || (signs && !aligned16(signs)) ||
      (workspace && !aligned16(workspace)))
    return KQ_EALIGN;
  if (!kq::gemm_shape_supported(M, N, K)) return KQ_EUNSUPPORTED;
  const int64_t need = kq::gemm_workspace_bytes(fmt, M, N, K, block_len, x_dt == KQ_BF16, signs);
  const bool uses_ws = block_len > 0 || signs || x_dt != KQ_BF16 || kq::gemm_split_count(fmt, M, N, K) > 1;
  if (uses_ws && (!workspace || (int64_t)ws_bytes < need)) return KQ_EWORKSPACE;
  return launched(kq::launch_gemm(fmt, packed, N, K, x, x_dt == KQ_BF16, M, block_len, signs, y,
                                  workspace, as_stream(stream)));
}

}  // extern "C"
