"""CPU fp64 oracle (test infrastructure only; never imported by the product path)."""
