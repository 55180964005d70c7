"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, orc):
    pin(orc)


def test_argument_validation(orc):
    import numpy as np
    A = np.zeros((4, 8), np.float16)
    B = np.zeros((3, 8), np.float16)
    with pytest.raises(ValueError):
        orc.gemm(A, B, K=9)          # K > lda
    with pytest.raises(ValueError):
        orc.gemm_sample(A, B, [4], [0])   # row out of range
    with pytest.raises(ValueError):
        orc.gemv_m1(np.zeros(8, np.float16), B, K=9)
