"""The CPU oracle against the pages' definitions, printed numbers and closed
forms (no GPU)."""
import pytest

import oracle.paged_attention_ref as ref
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ref)
