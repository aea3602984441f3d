"""CPU oracle (test infrastructure only): see kvarn_oracle."""
