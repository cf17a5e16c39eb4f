"""CPU oracle of the MoE layer (test infrastructure only: used by the tests,
the package smoke check and the benchmark's CPU-baseline leg; never by the
library's own path)."""
