"""CPU oracle of the MXFP4 routed-expert MoE layer (test infrastructure only)."""
