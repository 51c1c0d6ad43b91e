"""Measurement-only probes: hardware ceilings (ceilings.hip) and per-workgroup
phase timing of an instrumented copy of the kernels (phases.py)."""
