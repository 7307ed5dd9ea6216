"""CPU oracle of the ternary BitLinear forward path (test infrastructure only:
imported by tests/, the smoke check and the benchmark's CPU-baseline leg)."""
