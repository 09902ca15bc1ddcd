"""CPU oracle for the sparse global attention forward pass (test infrastructure only)."""
