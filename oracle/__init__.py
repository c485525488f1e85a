"""CPU float64 oracle (test infrastructure; see oracle.py)."""
