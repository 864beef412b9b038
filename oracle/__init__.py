"""CPU oracle for the PowerSGD compression step (test infrastructure only)."""
