"""Seeded synthetic workloads and the drivers that run them for measurement.

Not part of the attention library: ``inputs`` generates the inputs that the
tests, the smoke check and the benchmark share (no attention arithmetic in
it); ``profile_run`` and ``trace_run`` run one workload under a profiler or
with the per-workgroup timeline switched on.
"""
