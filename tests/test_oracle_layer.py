"""Pins of the oracle's arithmetic (CPU only): brute force, library routines, closed forms
and the article's invariants.  The checks live in tests/oracle_pins.py."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


def test_softmax_brute_force_worked_geometry():
    oracle_pins.check_softmax_brute_force("worked_f15_c1_table.json", T=2, H=1, d=4, L=1)


def test_linear_closed_form_worked_geometry():
    oracle_pins.check_linear_closed_form("worked_f15_c1_table.json", T=2, H=2, d=4, L=3)


def test_membership_probe_worked_geometry():
    oracle_pins.check_membership_probe("worked_f15_c1_table.json", T=3, L=2)
