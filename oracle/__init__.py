"""fp64 CPU oracle of the Mamba-3 SSM recurrence (test infrastructure only)."""
