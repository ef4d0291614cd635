"""CPU oracle for the verify step (test infrastructure; see verify_oracle)."""
