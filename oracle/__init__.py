"""fp64 CPU oracle for SWA(w,s) attention -- test infrastructure only (see oracle.py)."""
