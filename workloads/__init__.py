"""Seeded synthetic inputs and workload shapes, shared by the tests, the smoke check and the
benchmark.  This package only draws random tensors of given shapes; it computes nothing the
method defines (no compression, rotation, scoring, selection or quantization arithmetic)."""
