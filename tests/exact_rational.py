"""Exact-rational brute force for tiny groups (a pin on the oracle, not part of it).

Everything is computed with ``fractions.Fraction``: the binary16 scale values
come from numpy's own float16 decoding, the quotient w/s is exact, rounding is
Python's round-half-even on a Fraction, and the objective is summed exactly.
It follows the definition on the CliffQuant README ("What CliffQuant changes"):
min over positive finite binary16 s of max_e sum_i d_ei (w_i - s q_i(s))^2 with
q_i = clip(round-half-even(w_i/s), -8, 7) and the lower bit pattern on a tie.
Only the nonzero weights are passed in: a zero weight has code 0 and error 0 at
every scale.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

BITS = np.arange(0x0001, 0x7C00, dtype=np.uint16)
SCALES = [Fraction(float(v)) for v in BITS.view(np.float16).astype(np.float64)]


def code(w: Fraction, s: Fraction) -> int:
    q = round(w / s)  # Fraction.__round__: nearest integer, halves to even
    return max(-8, min(7, q))


def env_errors(ws, ds, s):
    qs = [code(w, s) for w in ws]
    return [sum((d * (w - s * q) ** 2 for w, d, q in zip(ws, de, qs)), Fraction(0)) for de in ds]


def solve(weights, diagonals):
    """Exact (bits, F_min, F_runner_up, all F) for nonzero float32 weights and diagonals [E][n]."""
    ws = [Fraction(float(np.float32(x))) for x in weights]
    ds = [[Fraction(float(np.float32(x))) for x in row] for row in diagonals]
    Fs = [max(env_errors(ws, ds, s)) for s in SCALES]
    order = sorted(range(len(Fs)), key=lambda j: (Fs[j], j))
    best, second = order[0], order[1]
    return int(BITS[best]), Fs[best], Fs[second], Fs
