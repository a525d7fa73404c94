"""CPU oracle for SAS gated block-sparse attention (test infrastructure only)."""
