"""CPU oracle (test infrastructure only; see mbq_oracle.py)."""
