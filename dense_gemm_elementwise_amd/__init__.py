"""Fused fp16 GEMM + elementwise epilogue for AMD MI355X (gfx950)."""
