"""CPU oracle (test infrastructure only; see far_oracle's module docstring)."""
