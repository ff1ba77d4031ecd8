"""Checks of the oracle against values printed on the source pages (CPU only)."""

import os

import numpy as np

from oracle import e4m3

HERE = os.path.join(os.path.dirname(__file__), "golden")


def load_ints(name):
    rows = [l.strip() for l in open(os.path.join(HERE, name)) if l.strip() and not l.startswith("#")]
    return np.array([int(r) for r in rows], dtype=np.float64)


def test_printed_exact_integers_round_trip():
    v = load_ints("e4m3_exact_ints.txt")
    assert np.array_equal(e4m3.decode(e4m3.encode(v)), v)
    assert np.array_equal(e4m3.decode(e4m3.encode(-v)), -v)


def test_integers_between_printed_ranges_are_not_exact():
    # the ranges change step exactly where the e4m3 grid spacing doubles
    for x in (17.0, 19.0, 33.0, 34.0, 35.0, 37.0, 62.0):
        assert e4m3.decode(e4m3.encode(np.array([x])))[0] != x
