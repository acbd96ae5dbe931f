"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle and its loader (see oracle.py)."""
