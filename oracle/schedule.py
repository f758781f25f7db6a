"""Reference schedules (test infrastructure only, like the rest of the oracle).

Written from the ResidualKV review page, section 2.6 (fixed and dynamic stride):

* fixed stride: a reference every s tokens;
* dynamic stride: the gap grows with the position,
      p_{m+1} = p_m + s_0 + floor(alpha (p_m - n_sink)),   p_0 = n_sink,
  and, ignoring the floor, the number of references up to T is about
      log_{1 + alpha}(1 + alpha (T - n_sink) / s_0)
  (alpha = 0 is the fixed stride, the limit of that expression: (T - n_sink) / s_0).

Readings where the page is silent:
* alpha is a decimal the caller writes down (0.001, 0.02, ...); the floor is taken
  of the exact product, so alpha is held as a rational (fractions.Fraction of the
  decimal string) and the recurrence runs in Python integers;
* the n_sink tokens before p_0 have no earlier token to be compared with, so they
  are stored directly as references as well;
* references are placed at positions below a caller-given limit. Table VI's
  counts at 262K (26,189 / 3,354 / 319 / 149 / 83 for alpha = 0 / 0.001 / 0.02 /
  0.05 / 0.1, s_0 = 10) are all reproduced with n_sink = 0 and a limit of
  262144 - 256, i.e. no reference among the last 256 positions.

Parity: pinned by tests/test_oracle_schedule.py (Table VI, the fixed-stride special
case, a hand-derived small case, the exact floor at integer products, and the
closed form's approximation).
"""

from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Union

Alpha = Union[str, int, Fraction]


def as_fraction(alpha: Alpha) -> Fraction:
    """alpha as an exact rational; a float is read through its shortest decimal."""
    if isinstance(alpha, float):
        alpha = repr(alpha)
    a = Fraction(alpha)
    if a < 0:
        raise ValueError("alpha must be >= 0")
    return a


def dynamic_reference_positions(limit: int, s0: int, n_sink: int, alpha: Alpha) -> List[int]:
    """Sorted reference positions below `limit` (section 2.6, dynamic stride)."""
    if s0 < 1 or n_sink < 0 or limit < 0:
        raise ValueError("s0 >= 1, n_sink >= 0, limit >= 0")
    a = as_fraction(alpha)
    out = list(range(min(n_sink, limit)))  # sink tokens: stored directly
    p = n_sink
    while p < limit:
        out.append(p)
        # floor of the exact product (Fraction floor division rounds toward -inf)
        p = p + s0 + math.floor(a * (p - n_sink))
    return out


def fixed_reference_positions(limit: int, s: int) -> List[int]:
    """Every s-th position from 0 (section 2.6, fixed stride)."""
    return list(range(0, max(limit, 0), s))


def approx_reference_count(T: float, s0: int, n_sink: int, alpha: Alpha) -> float:
    """The page's continuous approximation of the number of references up to T
    (section 2.6); alpha = 0 takes its limit (T - n_sink) / s0."""
    a = float(as_fraction(alpha))
    x = (T - n_sink) / s0
    if a == 0.0:
        return x
    return math.log1p(a * x) / math.log1p(a)
