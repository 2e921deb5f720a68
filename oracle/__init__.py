"""fp64 CPU oracle of the JSSA decode step (test infrastructure only)."""
