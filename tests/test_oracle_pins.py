"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


def test_gather_probe_fp32_pool():
    oracle_pins.pin_gather_probe(state_dtype="f32")


def test_output_shape():
    import oracle
    assert oracle.fwd_output_shape((37, 8192), (512, 32, 128, 128)) == (37, 4096)
