"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)


def test_golden_has_citations():
    rows = oracle_pins.read_golden()
    assert len(rows) >= 3
    for name, _, _, cite in rows:
        assert "Tutti reading notes" in cite and "eq." in cite or "step" in cite, name
