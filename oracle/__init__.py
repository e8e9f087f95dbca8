"""CPU oracle for the batch-invariant token-logprob path (test infrastructure only)."""
