"""CPU oracle (test infrastructure only; see twnorm_oracle's header)."""
