"""Pins of the oracle's rab bucketiser (CPU only)."""
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.BUCKET_PINS, ids=lambda p: p.__name__)
def test_bucket_pins(pin):
    pin(oracle)
