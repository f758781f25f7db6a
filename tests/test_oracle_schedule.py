"""Pins of the oracle's reference schedules (ResidualKV review page, section 2.6,
and Table VI in section 4.6)."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.schedule import (
    approx_reference_count,
    as_fraction,
    dynamic_reference_positions,
    fixed_reference_positions,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")


def table6():
    return json.load(open(GOLDEN))["table6_reference_counts"]


def test_table6_counts_at_262k():
    """All five printed counts, with n_sink = 0 and no reference among the last
    256 positions (the reading under which the table is reproduced)."""
    t = table6()
    for a, want, pct in zip(t["alpha"], t["references"], t["printed_percent"]):
        pos = dynamic_reference_positions(t["T"] - 256, t["s0"], 0, a)
        assert len(pos) == want, a
        assert round(100.0 * len(pos) / t["T"], 2) == pct, a


def test_table6_needs_the_tail_window():
    """Without the window only alpha >= 0.02 match: the fixed stride from 0 to 262144
    gives ceil(262144 / 10) = 26,215 references, not the printed 26,189, and
    alpha = 0.001 gives 3,355, not 3,354."""
    t = table6()
    full = [len(dynamic_reference_positions(t["T"], t["s0"], 0, a)) for a in t["alpha"]]
    assert full[0] == math.ceil(t["T"] / t["s0"]) == 26215
    assert full[1] == t["references"][1] + 1
    assert full[2:] == t["references"][2:]


def test_alpha_zero_is_the_fixed_stride():
    for limit, s in [(0, 10), (1, 10), (37, 3), (1000, 10), (4099, 16)]:
        assert dynamic_reference_positions(limit, s, 0, "0") == fixed_reference_positions(limit, s)
        assert fixed_reference_positions(limit, s) == list(np.arange(0, limit, s))


def test_hand_derived_small_case():
    # s0 = 3, n_sink = 2, alpha = 1/2: sinks 0, 1; then 2; 2+3+0 = 5; 5+3+1 = 9;
    # 9+3+3 = 15; 15+3+6 = 24; 24+3+11 = 38; 38+3+18 = 59 >= 40 stops.
    assert dynamic_reference_positions(40, 3, 2, "0.5") == [0, 1, 2, 5, 9, 15, 24, 38]
    assert dynamic_reference_positions(38, 3, 2, "1/2") == [0, 1, 2, 5, 9, 15, 24]
    assert dynamic_reference_positions(1, 3, 2, "0.5") == [0]
    assert dynamic_reference_positions(0, 3, 2, "0.5") == []


def test_floor_is_exact_at_integer_products():
    # alpha = 0.29: 0.29 * 100 is 28.999999999999996 in binary floating point, but the
    # exact product is 29, so the gap after position 100 is s0 + 29.
    assert math.floor(0.29 * 100) == 28
    pos = dynamic_reference_positions(300, 100, 0, "0.29")
    assert pos == [0, 100, 229]
    assert dynamic_reference_positions(300, 100, 0, 0.29) == pos  # a float is read as its decimal
    assert as_fraction(0.29) == Fraction(29, 100)


def test_gaps_follow_the_recurrence():
    for a in ["0.001", "0.02", "0.1", "3/7"]:
        f = Fraction(a)
        pos = dynamic_reference_positions(200000, 7, 5, a)
        assert pos[:5] == [0, 1, 2, 3, 4]
        dyn = pos[5:]
        assert dyn[0] == 5
        for p, q in zip(dyn, dyn[1:]):
            assert q - p == 7 + (f.numerator * (p - 5)) // f.denominator
        assert dyn[-1] < 200000 <= dyn[-1] + 7 + (f.numerator * (dyn[-1] - 5)) // f.denominator


def test_closed_form_tracks_the_count():
    """The page's log approximation ignores the floor, which only shortens gaps, so
    the recurrence places at least as many references; at Table VI's alphas the
    two stay within 2 %."""
    t = table6()
    for a in t["alpha"][1:]:
        n = len(dynamic_reference_positions(t["T"], t["s0"], 0, a))
        approx = approx_reference_count(t["T"], t["s0"], 0, a)
        assert n >= approx - 1
        assert abs(n - approx) / n < 0.02, (a, n, approx)
    # growth is logarithmic: doubling T adds about log(2) / log(1 + alpha) references
    n1 = len(dynamic_reference_positions(1 << 20, 10, 0, "0.1"))
    n2 = len(dynamic_reference_positions(1 << 21, 10, 0, "0.1"))
    assert abs((n2 - n1) - math.log(2) / math.log(1.1)) <= 2


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        dynamic_reference_positions(10, 0, 0, "0.1")
    with pytest.raises(ValueError):
        dynamic_reference_positions(10, 1, -1, "0.1")
    with pytest.raises(ValueError):
        dynamic_reference_positions(10, 1, 0, "-0.1")
