"""fp64 CPU oracle of the q4gsw linear layer (test infrastructure only)."""
