// kq_launch.h -- host-side launch entry points between the C ABI (api.hip)
// and the kernels.  Shapes reaching these functions are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

constexpr int kFmtPQ2 = 1;
constexpr int kFmtQ8 = 2;

inline int group_of(int fmt) { return fmt == kFmtPQ2 ? 128 : 32; }

// Planar packed buffer: qs plane, then the fp16 d plane at a 256-B boundary.
struct PlanarView {
  uint8_t* qs;
  uint8_t* d;
  int64_t qs_bytes;      // code plane: whole 16-row tiles, ceil(N/16)*16 * row_bytes
  int64_t row_bytes;     // code bytes per row (32 per block)
  int64_t d_per_row;     // scales per row (blocks)
  int64_t d_chunks;      // scale chunks of 8 blocks per 16-row tile, ceil(d_per_row / 8)
  int64_t d_tile_bytes;  // scale bytes per 16-row tile, 256 * d_chunks
  int64_t total_bytes;
};

inline PlanarView planar_view(int fmt, int64_t N, int64_t K, void* base) {
  PlanarView v;
  v.row_bytes = fmt == kFmtPQ2 ? K / 4 : K;
  v.qs_bytes = (N + 15) / 16 * 16 * v.row_bytes;
  int64_t d_off = (v.qs_bytes + 255) / 256 * 256;
  v.d_per_row = K / group_of(fmt);
  v.d_chunks = (v.d_per_row + 7) / 8;
  v.d_tile_bytes = 256 * v.d_chunks;
  v.total_bytes = d_off + (N + 15) / 16 * v.d_tile_bytes;
  v.qs = (uint8_t*)base;
  v.d = (uint8_t*)base + d_off;
  return v;
}

// All return 0 on success, -1 if the HIP runtime rejected a launch (launch_gemv
// and launch_gemv_multi: -2 if no launch plan fits the arguments).
int launch_pack(int fmt, const float* W, int64_t N, int64_t K, void* packed, hipStream_t st);
int launch_unpack(int fmt, const void* packed, int64_t N, int64_t K, float* W, hipStream_t st);
int launch_transcode_ptq1(const void* ptq1, int64_t N, int64_t K, void* packed, hipStream_t st);
int launch_hadamard(const void* x, int x_bf16, void* xr, int xr_bf16, int64_t M, int64_t K,
                    int n, const int8_t* signs, hipStream_t st);

// GEMV plan: how K is split across workgroups and how the grid is shaped.
struct GemvPlan {
  int split;      // S >= 1 K-slices (grid.y); < 1 if no plan fits
  int epl;        // PQ2_0 prologue: activation elements per lane (8 or 16)
  int gs;         // groups per wave
  int units;      // groups per rotation block (slices hold whole blocks)
  int nw;         // waves per workgroup
  int grid_x;     // workgroups along the rows
  int total_rb;   // 16-row blocks
  int lds_bytes;  // dynamic LDS per workgroup
  bool dalign;    // per-wave scale runs start on a 4-byte boundary
  bool few;       // PQ2_0: every workgroup's row blocks are in flight at once
};
GemvPlan plan_gemv(int fmt, int64_t M, int64_t N, int64_t K, int block_len, int split_req);
int64_t gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int block_len, int split_req);
int launch_gemv(int fmt, const void* packed, int64_t N, int64_t K, const float* x, int64_t M,
                int block_len, const int8_t* signs, int split_req, float* y, void* ws,
                hipStream_t st);

// Several weight sets (same K and format) times one activation: one launch,
// the workgroups split between the sets in proportion to their rows.
constexpr int kMaxSets = 4;
// 0 when a launch plan exists, -2 when none fits (as launch_gemv)
int check_gemv_multi(int fmt, int nsets, const int64_t* N, int64_t K, int64_t M, int block_len);
int launch_gemv_multi(int fmt, int nsets, const void* const* packed, const int64_t* N, int64_t K,
                      const float* x, int64_t M, int block_len, const int8_t* signs,
                      float* const* y, hipStream_t st);

// Largest K the prefill GEMM takes: a 256-row activation tile (256 * K * 2
// bytes) stays a 32-bit buffer range well below the out-of-range offset.
// gemm_shape_supported also bounds the tile count by an int.
constexpr int64_t kGemmMaxK = int64_t(1) << 21;
bool gemm_shape_supported(int64_t M, int64_t N, int64_t K);
// Loads-only twin of launch_gemv (same plan and weight loads, no arithmetic);
// -2 when kq_gemv has no plan for the arguments.
int launch_gemv_loads_twin(int fmt, const void* packed, int64_t N, int64_t K, const float* x,
                           int64_t M, int block_len, int split_req, uint32_t* sink, hipStream_t st);
// Streaming read of `bytes` (a multiple of 16) at buf: layout 0 grid-stride,
// 1 one contiguous chunk per workgroup.
int launch_probe_read(const void* buf, size_t bytes, int layout, int grid, int block,
                      uint32_t* sink, hipStream_t st);

int64_t gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int block_len, int x_bf16,
                             const void* signs_hint);
// K slices of the GEMM (1: one pass; more: fp32 partials in the workspace)
int gemm_split_count(int fmt, int64_t M, int64_t N, int64_t K);
// y[i] = sum_{s < S} part[s n + i], ascending s (the GEMV's split-K reduce)
int launch_splitk_reduce(const float* part, float* y, int64_t n, int S, hipStream_t st);
int launch_gemm(int fmt, const void* packed, int64_t N, int64_t K, const void* x, int x_bf16,
                int64_t M, int block_len, const int8_t* signs, float* y, void* ws, hipStream_t st);

}  // namespace kq
