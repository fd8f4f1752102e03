"""Plain CPU oracle of the prefill routed-expert product (test infrastructure only)."""
