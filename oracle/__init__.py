"""CPU oracle package (test infrastructure only; see uocr_oracle.py)."""
