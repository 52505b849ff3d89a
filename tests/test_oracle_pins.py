"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


def test_oracle_rejects_bad_arguments(o):
    import numpy as np
    with pytest.raises(RuntimeError):
        o.search(np.zeros((4, 3), np.float32), np.zeros((1, 3), np.float32), 5)  # k > n
    with pytest.raises(RuntimeError):
        o.topk(np.zeros(4, np.int32), 0)


def test_oracle_thread_count_positive(o):
    assert o.num_threads() >= 1
