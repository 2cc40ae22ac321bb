"""Fused GEMM + reduce-scatter epilogue + flag-gated reduce for MI355X."""
