"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_inputs(orc):
    import numpy as np

    pool = oracle.Pool.hnd(oracle.F32, 3, 16, 1, 4)
    kc = np.zeros(3 * 16 * 4, np.float32)
    vc = kc.copy()
    kn = np.zeros((1, 1, 4), np.float32)
    # page 0 is reserved and page 3 does not exist
    for page in (0, 3):
        with pytest.raises(oracle.OracleError):
            orc.append(pool, kc, vc, kn, kn, np.array([[page]], np.int32), np.array([0], np.int32))
    # more tokens than the table has blocks for
    with pytest.raises(oracle.OracleError):
        orc.append(pool, kc, vc, kn, kn, np.array([[1]], np.int32), np.array([16], np.int32))
    # causal prefill needs q_len <= kv_len
    q = np.zeros((2, 1, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        orc.prefill(pool, q, kc, vc, np.array([[1]], np.int32), np.array([1], np.int32),
                    np.array([0, 2], np.int32), 1.0, causal=True)
