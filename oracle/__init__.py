"""Float64 CPU oracle of the SpargeAttn hot path (test infrastructure only)."""
