"""Seeded synthetic workloads shared by the oracle tests, the GPU parity tests and the benchmark.

This package holds only random-number generation, shapes and dtype conversion. None of the
PowerSGD arithmetic lives here.
"""
from .synth import *  # noqa: F401,F403
