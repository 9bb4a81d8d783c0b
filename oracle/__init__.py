"""Plain CPU oracle for the block-quantized GEMM path (test infrastructure only)."""
