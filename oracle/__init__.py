"""fp64 CPU oracle of the sparse-MoE FFN forward -- test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import it."""
