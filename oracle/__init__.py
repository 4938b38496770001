"""CPU oracle for the routed-expert MoE layer (test infrastructure only)."""
