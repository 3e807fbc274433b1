"""CPU oracle of the RAT+ layer (test infrastructure only; see oracle.c)."""
