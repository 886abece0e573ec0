"""CPU oracle of the decode step (test infrastructure only; see oracle.py)."""
