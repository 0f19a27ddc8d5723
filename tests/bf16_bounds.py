"""Where a float32 computation rounded to bf16 may land, given the exact value.

The step normalises q and k in float32 and rounds them to bf16 (round to
nearest, ties to even). With u the exact (float64) normalised value and u32
the float32 one, |u32 - u| <= delta |u|, so the bf16 result is always one of
the two bf16 values that bracket u, and it is the one round-to-nearest gives
for u itself unless u lies within delta |u| of the midpoint between them.

delta for x / sqrt(sum x_i^2 + eps) over d terms in float32 (unit roundoff
2^-24; every operation below is counted at 2 units to cover a sqrt or divide
that is not correctly rounded):
* the sum of d squares (one rounding per product-add): relative error at most
  d 2^-24 / (1 - d 2^-24); the square root halves it;
* adding eps: 2^-24; square root: 2^-23; reciprocal: 2^-23; multiply: 2^-24.
Together (d / 2 + 6) 2^-24 to first order; (d / 2 + 8) 2^-24 is used.
"""
from __future__ import annotations

import numpy as np


def fp32_unit_rel_bound(d: int) -> float:
    return (d / 2 + 8) * 2.0 ** -24


def bf16_neighbours(u):
    """(lo, hi): the largest bf16 value <= u and the smallest >= u (float64)."""
    u = np.asarray(u, dtype=np.float64)
    _, e = np.frexp(u)                      # u = m 2^e, 0.5 <= |m| < 1
    ulp = np.ldexp(1.0, e - 8)              # bf16: 8 significant bits
    lo = np.floor(u / ulp) * ulp
    hi = np.ceil(u / ulp) * ulp
    return lo, hi


def check_rounded(k_bf16, u, rel_bound):
    """Compare bf16 values (as float) with the exact values they round.

    Returns (all_bracketing, all_exact_outside_band, n_band, n_differ): every
    element is one of the two bf16 neighbours of u; every element farther
    than rel_bound |u| from their midpoint equals round-to-nearest(u); how
    many elements lie inside that band; how many differ from round-to-nearest(u).
    """
    k = np.asarray(k_bf16, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    lo, hi = bf16_neighbours(u)
    mid = 0.5 * (lo + hi)
    rne = np.where(u < mid, lo, hi)         # (an exact tie falls inside the band)
    band = (lo != hi) & (np.abs(u - mid) <= rel_bound * np.abs(u))
    bracket = (k == lo) | (k == hi)
    exact = band | (k == rne)
    return bool(bracket.all()), bool(exact.all()), int(band.sum()), int((k != rne).sum())
