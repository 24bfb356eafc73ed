"""The CPU oracle against facts outside itself (see tests/oracle_pins.py)."""
import pytest

import oracle.candidates
import oracle.prefill
import oracle.indexer_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    O.candidates = oracle.candidates  # the pins reach the candidate oracle as O.candidates
    O.prefill = oracle.prefill
    fails = pin(O)
    assert not fails, "\n".join(fails[:10])
