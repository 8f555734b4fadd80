"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_threads_do_not_change_results(orc):
    import numpy as np
    rng = np.random.default_rng(3)
    c = oracle_pins._rand_case(rng, 3, 33, 7, 5)
    a, la = orc.scan_fwd(nthreads=1, **c)
    b, lb = orc.scan_fwd(nthreads=5, **c)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_empty_sequence_gives_zero_state(orc):
    import numpy as np
    x = np.zeros((2, 0, 3))
    out, last = orc.scan_fwd(x, x, -np.ones((3, 4)), np.zeros((2, 0, 4)), np.zeros((2, 0, 4)))
    assert out.shape == (2, 0, 3) and np.array_equal(last, np.zeros((2, 3, 4)))
