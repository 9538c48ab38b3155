"""tiled_matmul_amd: an MI355X (gfx950) bf16 GEMM C = A * B^T behind a C-ABI library."""
