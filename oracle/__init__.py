"""CPU oracle for the PRR hot path (test infrastructure only; see prr_oracle.py)."""
