"""Block-quantized decode matmuls for MI355X (gfx950)."""
