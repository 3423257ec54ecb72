"""The CPU oracle against its pins (worked examples, exact arithmetic, closed
forms, invariants and independent libraries).  No GPU."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_oracle_rejects_bad_arguments(oracle_lib):
    import numpy as np
    import oracle
    lib = oracle_lib
    x = np.zeros(4, np.float32)
    y = np.zeros(4)
    P = lambda a: a.ctypes.data
    assert lib.oracle_pointwise_chain(P(x), P(x), P(x), -1, 0.5, 0, P(y)) != 0
    assert lib.oracle_pointwise_chain(P(x), P(x), P(x), 4, 0.5, 7, P(y)) != 0
    assert lib.oracle_pointwise_chain(None, None, None, 0, 0.5, 0, None) == 0
    assert lib.oracle_row_mean_epilogue(P(x), P(x), P(x), P(x), 1, 0, 1.1, 0.1, 0, P(y)) != 0
    assert lib.oracle_add_layernorm_gelu(5, P(x), None, P(x), P(x), 1, 4, 1e-5, 0, 0, P(y)) != 0
    assert lib.oracle_add_layernorm_gelu(0, P(x), None, P(x), P(x), 0, 4, 1e-5, 0, 0, P(y)) == 0
    with pytest.raises(ValueError):
        oracle.row_mean_epilogue(np.zeros((2, 3), np.float32), x, x, x)
