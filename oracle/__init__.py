"""CPU oracle (test infrastructure only): see eagle3_oracle.py's header."""
