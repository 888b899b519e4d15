"""One tensor-parallel rank's share of a Megatron-style layer on MI355X."""
