"""The backward oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import pins_bwd


@pytest.mark.parametrize("name,pin", pins_bwd.ALL_PINS, ids=[n for n, _ in pins_bwd.ALL_PINS])
def test_backward_oracle_pin(name, pin):
    pin(oracle.bwd)


def test_backward_oracle_kl_zero_gives_zero_dq():
    import numpy as np
    q = np.zeros((1, 1, 3, 4), np.uint16)
    k = np.zeros((1, 1, 0, 4), np.uint16)
    L = np.full((1, 1, 3), -np.inf, np.float32)
    dQ, dK, dV = oracle.bwd(q, k, k, None, L, q, 1, 1, 1, 3, 0, 4, 0.5, False)
    assert dQ.shape == (1, 1, 3, 4) and np.all(dQ == 0) and dK.size == 0 and dV.size == 0


@pytest.mark.parametrize("name,pin", pins_bwd.SINK_PINS, ids=[n for n, _ in pins_bwd.SINK_PINS])
def test_backward_sink_oracle_pin(name, pin):
    pin(oracle.bwd, oracle.bwd_sinks)


@pytest.mark.parametrize("name,pin", pins_bwd.GIVEN_O_PINS,
                         ids=[n for n, _ in pins_bwd.GIVEN_O_PINS])
def test_backward_given_o_oracle_pin(name, pin):
    pin(oracle.bwd)


def test_backward_given_o_needs_o():
    import numpy as np
    q = np.zeros((1, 1, 3, 4), np.uint16)
    L = np.zeros((1, 1, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.bwd(q, q, q, None, L, q, 1, 1, 1, 3, 3, 4, 0.5, False, O=np.zeros(5, np.float32))
