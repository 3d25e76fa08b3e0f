"""Float64 CPU oracle (test infrastructure only; never on the product path)."""
