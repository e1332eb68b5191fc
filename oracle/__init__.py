"""CPU oracle for the MoE feed-forward layer: test infrastructure only (see moe_oracle.c)."""
