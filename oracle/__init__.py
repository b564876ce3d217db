"""fp64 CPU oracle of the LISA layer -- test infrastructure only (see oracle.py)."""
