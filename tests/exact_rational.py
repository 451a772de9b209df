"""Exact-rational brute force for tiny groups (a pin on the oracle, not part of it).

Everything is computed with ``fractions.Fraction``: the binary16 scale values
come from numpy's own float16 decoding, the quotient w/s is exact, rounding is
Python's round-half-even on a Fraction, and the objectives are summed exactly.
It follows the definition on the CliffQuant README ("What CliffQuant changes"):
min over positive finite binary16 s of max_e sum_i d_ei (w_i - s q_i(s))^2 with
q_i = clip(round-half-even(w_i/s), qmin, qmax) and the lower bit pattern on a
tie; the pooled policy (the README's opening question: average the environments
first) minimises (1/E) sum_e of the same per-environment sums.  The code range
is the README's "Use the solver" quantizer specification (qmin, qmax).
Only the nonzero weights are passed in: a zero weight has code 0 and error 0 at
every scale.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

BITS = np.arange(0x0001, 0x7C00, dtype=np.uint16)
SCALES = [Fraction(float(v)) for v in BITS.view(np.float16).astype(np.float64)]


def code(w: Fraction, s: Fraction, qmin: int = -8, qmax: int = 7) -> int:
    q = round(w / s)  # Fraction.__round__: nearest integer, halves to even
    return max(qmin, min(qmax, q))


def env_errors(ws, ds, s, qmin=-8, qmax=7):
    qs = [code(w, s, qmin, qmax) for w in ws]
    return [sum((d * (w - s * q) ** 2 for w, d, q in zip(ws, de, qs)), Fraction(0)) for de in ds]


class Exact:
    """Argmin bits, minimum and runner-up of the minimax (F) and pooled (P) objectives."""

    def __init__(self, Fs, Ps):
        self.F, self.P = Fs, Ps
        self.mm_bits, self.F1, self.F2 = self._best(Fs)
        self.pl_bits, self.P1, self.P2 = self._best(Ps)

    @staticmethod
    def _best(vals):
        order = sorted(range(len(vals)), key=lambda j: (vals[j], j))
        return int(BITS[order[0]]), vals[order[0]], vals[order[1]]

    def __iter__(self):  # (bits, F1, F2, all F): the minimax result as a tuple
        return iter((self.mm_bits, self.F1, self.F2, self.F))


def solve(weights, diagonals, qmin: int = -8, qmax: int = 7) -> Exact:
    """Exact results for nonzero float32 weights and diagonals [E][n] over every binary16 scale."""
    ws = [Fraction(float(np.float32(x))) for x in weights]
    ds = [[Fraction(float(np.float32(x))) for x in row] for row in diagonals]
    E = len(ds)
    Fs, Ps = [], []
    for s in SCALES:
        fe = env_errors(ws, ds, s, qmin, qmax)
        Fs.append(max(fe))
        Ps.append(sum(fe, Fraction(0)) / E)
    return Exact(Fs, Ps)
