"""The float64 oracle against closed forms, invariants, hand values and page facts."""

import pytest

import oracle.adamw as oa
import oracle.muon as om
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_ORACLE_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(om)


def test_page_hyperparameters():
    oc.check_page_hyperparameters()


@pytest.mark.parametrize("check", oc.ADAMW_CHECKS, ids=lambda f: f.__name__)
def test_adamw_oracle_pin(check):
    check(oa)
