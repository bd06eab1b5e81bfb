"""fp64 CPU oracle of the MoE layer.  Test infrastructure: imported only by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the library."""
