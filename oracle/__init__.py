"""Float64 CPU oracle for fused alpha-entmax attention (test infrastructure only)."""
