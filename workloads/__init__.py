"""Seeded synthetic workloads for the speculative-decoding verify step.

Shared by the tests, the benchmark and the smoke check.  Holds input
generation only (tree shapes, lengths, random tensors and draft tokens); it
contains none of the verify method's arithmetic.
"""
from .gen import CONFIGS, CONFIG_ORDER, Workload, make  # noqa: F401
from . import drafts, heads, masks, trees  # noqa: F401
