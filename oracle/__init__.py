"""CPU oracle of the W1.58A8 BitLinear: test infrastructure only (see oracle.py)."""
