"""fp64 CPU oracle of the LatentMoE layer forward (test infrastructure only)."""
