"""Seeded synthetic inputs shared by the oracle and the device path.

Holds the workload structure (``spec``), the counter-based value generator
(``rng``) and, under ``csrc``, the same generator for device memory.  It holds
no part of the attention method.
"""
from . import rng, spec  # noqa: F401
