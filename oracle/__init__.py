"""fp64 CPU oracle for MSA main attention (test infrastructure only: used by
tests/, the smoke check and the CPU-baseline leg of the benchmark, never by
the product path)."""
