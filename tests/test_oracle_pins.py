"""The fp64 oracle against closed forms, library routines, brute force and invariants."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()


def test_grouping_must_divide_heads():
    import numpy as np

    import oracle
    assert [oracle.kv_head(h, 6, 2) for h in range(6)] == [0, 0, 0, 1, 1, 1]
    assert [oracle.kv_head(h, 4, 1) for h in range(4)] == [0, 0, 0, 0]
    for heads, kv_heads in ((6, 4), (4, 0), (3, 5)):
        with pytest.raises(ValueError):
            oracle.kv_head(0, heads, kv_heads)
    q = np.zeros((1, 6, 2, 2))
    with pytest.raises(ValueError):
        oracle.forward(q, np.zeros((1, 4, 2, 2)), np.zeros((1, 4, 2, 2)), 1.0, False)
