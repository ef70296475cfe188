"""fp64 CPU oracle (test infrastructure only; see kvq_oracle's header)."""
