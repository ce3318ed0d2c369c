"""The CPU oracle against its pins (no GPU)."""

import pytest

import oracle_pins as pins
from oracle import gather, gemm


@pytest.mark.parametrize("check", pins.GATHER_CHECKS, ids=lambda c: c.__name__)
def test_gather_oracle_pin(check):
    check(gather)


@pytest.mark.parametrize("check", pins.GEMM_CHECKS, ids=lambda c: c.__name__)
def test_gemm_oracle_pin(check):
    check(gemm)
