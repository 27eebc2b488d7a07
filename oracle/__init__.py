"""CPU oracle of the MSA forward pass (test infrastructure only; see msa_oracle)."""
