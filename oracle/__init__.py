"""Double-precision CPU oracle of the selective scan (test infrastructure only)."""
