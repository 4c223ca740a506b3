"""The oracle's triangle multiplication against its pins (CPU only)."""
import pytest

import oracle_trimul_pins


@pytest.fixture(scope="module")
def tref(oracle_lib):
    def _tref(a, w, dtype, direction):
        return oracle_lib.trimul(a, w, dtype=dtype, direction=direction, nthreads=4)
    return _tref


@pytest.mark.parametrize("pin", oracle_trimul_pins.ALL_TRIMUL_PINS, ids=lambda f: f.__name__)
def test_oracle_trimul_pin(tref, pin):
    pin(tref)
