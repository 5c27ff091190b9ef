"""CPU pins of the 8-bit KV oracle (oracle/quant.py and the quantised write
and decode built on it): OCP E4M3 fixed points, torch's independent float8
and rounding routines, brute force, round trips, lossless cases."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.QUANT_PINS, ids=[p.__name__ for p in P.QUANT_PINS])
def test_quant_pin(pin):
    pin()


@pytest.mark.parametrize("pin", P.TOKEN_PINS, ids=[p.__name__ for p in P.TOKEN_PINS])
def test_token_scale_pin(pin):
    pin()
