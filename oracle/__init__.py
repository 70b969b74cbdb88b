"""CPU oracle of the depth loop (test infrastructure only; see oracle.h)."""
