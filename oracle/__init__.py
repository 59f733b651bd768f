"""CPU oracle (test infrastructure only; see pk_oracle's header)."""
