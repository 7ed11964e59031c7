"""CPU oracle (test infrastructure only; see mq_oracle's header)."""
