"""The fp64 oracle against results the mathematics fixes (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_rejects_malformed_cu_seqlens(orc):
    q = np.zeros((4, 1, 2), np.float32)
    a = np.ones((4, 1), np.float32)
    for cu in ([1, 4], [0, 3], [0, 3, 2, 4]):
        with pytest.raises(ValueError):
            orc.prefill(q, q, q, a, a, cu_seqlens=np.array(cu, np.int32))


def test_threads_reported(orc):
    assert orc.threads_used(3) == 3
    assert orc.threads_used(0) >= 1


def test_thread_count_does_not_change_results(orc):
    rng = np.random.default_rng(5)
    T, H, d = 40, 6, 8
    q, k, v, a, b, S0 = pins.random_case(rng, T, H, d, d)
    o1, s1 = orc.prefill(q, k, v, a, b, S0=S0, threads=1)
    o4, s4 = orc.prefill(q, k, v, a, b, S0=S0, threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)
