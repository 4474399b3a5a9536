"""Parity tolerances shared by the tests.

ATOL is the bar the attention output must meet against the oracle (max-abs,
float32 output against the float64 oracle, bf16 or Q4 inputs upcast the same
way on both sides).

``gate`` is a tighter internal bar.  With N(0,1) inputs a decode output over L
tokens has magnitude about sqrt(e / L), so at 16k tokens a dropped block moves
it by ~2e-4, which ATOL alone would miss.  The device path keeps every input
exact and accumulates in float32; the values it forms and hands to bf16
operands -- a shifted consumer's rotated query, and in the matrix-core paths
the softmax weights -- go as bf16 hi + lo pairs, about 16 bits (some 2**-17
relative), so its error is float32 accumulation order plus that.  The gate
allows 1e-4 scaled by rms(out) * sqrt(L) (~1 for these inputs), and the
planted-mistake tests check that the mistakes one could plausibly make exceed
it.
"""
import numpy as np

ATOL = 2e-3


def gate(ref: np.ndarray, L: int) -> float:
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    return 1e-4 * max(1.0, rms * np.sqrt(max(L, 1)))
