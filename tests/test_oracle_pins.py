"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_golden_file_has_citation_and_cases():
    text = open(P.GOLDEN).read()
    assert "Intuizione Centrale" in text
    assert len(P.load_golden()) == 3
