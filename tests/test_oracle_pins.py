"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def ora():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(ora, pin):
    pin(ora)


def test_rejects_bad_shapes(ora):
    import numpy as np
    q = np.zeros((1, 6, 4))
    k = np.zeros((1, 4, 3, 4))
    with pytest.raises(ValueError):
        ora.decode(q, k, k, np.array([3], np.int32), 1.0)  # H % G != 0
    with pytest.raises(ValueError):
        ora.meanpool(np.zeros((2, 24), np.float32), 6, 4)


def test_thread_count_does_not_change_result(ora):
    import numpy as np
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 8, 16))
    k = rng.standard_normal((3, 2, 33, 16))
    v = rng.standard_normal((3, 2, 33, 16))
    lens = np.array([33, 17, 2], np.int32)
    a = ora.decode(q, k, v, lens, 0.25, nthreads=1)
    b = ora.decode(q, k, v, lens, 0.25, nthreads=7)
    assert np.array_equal(a, b)
