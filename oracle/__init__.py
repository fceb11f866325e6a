"""CPU oracle package (test infrastructure only; see pisa_oracle.py)."""
