"""fp64 CPU oracle for exact attention -- test infrastructure only (see oracle.py)."""
