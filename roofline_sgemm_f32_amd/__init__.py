"""MI355X (gfx950) single-precision dense matrix multiply, C = A * B."""
