"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle
import oracle_decode_pins
import oracle_pins
import oracle_rope_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("pin", oracle_rope_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_rope_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("pin", oracle_decode_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_decode_pin(pin):
    pin(oracle)


import oracle_varlen_pins  # noqa: E402


@pytest.mark.parametrize("pin", oracle_varlen_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_varlen_pin(pin):
    pin(oracle)


import oracle_masked_pins  # noqa: E402


@pytest.mark.parametrize("pin", oracle_masked_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_masked_pin(pin):
    pin(oracle)
