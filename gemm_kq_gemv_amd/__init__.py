"""gemm_kq_gemv_amd: quantized-weight GEMV / GEMM for MI355X (gfx950)."""
