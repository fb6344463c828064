"""CPU fp64 oracle for the fused attention forward pass (test infrastructure only)."""
