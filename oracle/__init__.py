"""fp64 CPU oracle of the ISPA hot path (test infrastructure only)."""
