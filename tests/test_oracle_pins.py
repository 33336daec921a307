"""The CPU oracle against the pages' numbers, a library routine, closed forms and invariances."""

import pytest

import oracle
from oracle import arith

from pins import ARITH_PINS, ORACLE_PINS


@pytest.mark.parametrize("pin", ARITH_PINS, ids=lambda p: p.__name__)
def test_arith_pin(pin):
    pin(arith)


@pytest.mark.parametrize("pin", ORACLE_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin, oracle_impl):
    pin(oracle_impl)


def test_oracle_source_is_test_infrastructure():
    with open(oracle.SOURCE) as f:
        head = f.read(600)
    assert "TEST INFRASTRUCTURE ONLY" in head
