"""CPU oracle (test infrastructure only; see oracle/kvc_oracle.c)."""
