"""fp64 CPU oracle for MLA prefill (test infrastructure only; never imported by the product path)."""
