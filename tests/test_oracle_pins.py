"""CPU pins of the oracle: every check in oracle_pins against the real build."""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.Bound()


@pytest.mark.parametrize("name,check", P.ALL_CHECKS, ids=[n for n, _ in P.ALL_CHECKS])
def test_pin(orc, name, check):
    check(orc)


def test_window_starts_by_hand():
    """Window starts worked out by hand from the definition (centered, shifted
    inward): T = 16, k = 3 (the 3D workload's time axis) and T = 8, k = 5."""
    assert [oracle.window_start(16, 3, 1, x) for x in range(16)] == [0, 0] + list(range(1, 14)) + [13]
    assert [oracle.window_start(8, 5, 1, x) for x in range(8)] == [0, 0, 0, 1, 2, 3, 3, 3]
    # dilation 2 on 10 positions: classes {0,2,4,6,8} and {1,3,5,7,9}, k = 3
    assert [oracle.window_start(10, 3, 2, x) for x in range(10)] == [0, 1, 0, 1, 2, 3, 4, 5, 4, 5]


def test_rejects_oversized_kernel():
    import numpy as np
    q = np.zeros((1, 5, 6, 1, 2))
    with pytest.raises(ValueError):
        oracle.na_fwd(q, q, q, (3, 3), (2, 1))   # H = 5 at d = 2 leaves a class of 2 < 3
