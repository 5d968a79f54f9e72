"""CPU oracle of the VSA2 attention layer (test infrastructure only)."""
