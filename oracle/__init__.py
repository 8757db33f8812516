"""CPU fp64 oracle (test infrastructure only; never used by the product path)."""
