"""Host schedules (momentum warm-up, NS coefficient tables) against the pages and hand values."""

import json
import os

import pytest

from muon_optimizer_step_amd import schedules as sch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def test_momentum_warmup_matches_the_page():
    facts = json.load(open(GOLDEN))
    start = facts["muon_momentum_warmup_start"]["value"]
    steps = facts["muon_momentum_warmup_steps"]["value"]
    end = facts["muon_momentum"]["value"]
    assert sch.muon_momentum(0) == pytest.approx(start, abs=1e-15)
    assert sch.muon_momentum(steps) == end and sch.muon_momentum(10 * steps) == end
    # halfway: (0.92 + 0.99) / 2 = 0.955; a tenth: 0.92 + 0.007 = 0.927
    assert sch.muon_momentum(750) == pytest.approx(0.955, abs=1e-15)
    assert sch.muon_momentum(150) == pytest.approx(0.927, abs=1e-15)
    vals = [sch.muon_momentum(t) for t in range(0, 2000, 7)]
    assert all(a <= b for a, b in zip(vals, vals[1:]))
    with pytest.raises(ValueError):
        sch.muon_momentum(-1)
    assert sch.muon_momentum(5, start=0.5, end=0.6, warmup_steps=0) == 0.6


def test_ns_coefficient_tables():
    assert sch.ns_coefficients(5) == [(3.4445, -4.7750, 2.0315)] * 5
    assert sch.ns_coefficients(0) == []
    t = [(1, 2, 3), (4, 5, 6)]
    assert sch.ns_coefficients(2, t) == [(1.0, 2.0, 3.0), (4.0, 5.0, 6.0)]
    for bad in ([(1, 2, 3)], [(1, 2), (3, 4)]):
        with pytest.raises(ValueError):
            sch.ns_coefficients(2, bad)
