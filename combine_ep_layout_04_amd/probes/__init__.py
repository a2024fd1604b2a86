"""Measurement kernels for the dispatch's access pattern (libep_probe.so),
used to attribute the bf16 dispatch's time; not part of the C ABI."""
