"""lossless_bit_weight_amd: W12 lossless 12-bit BF16 weights and small-M decode GEMM on MI355X."""
