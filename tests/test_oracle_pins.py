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


def test_tolerance_formulas():
    """The acceptance bounds: fp16 as stated; bf16 swaps half an fp16 ulp for
    half a bfloat16 ulp in the relative term."""
    import numpy as np
    import oracle
    c = np.array([0.0, 1.0, -10.0, 1000.0])
    assert np.allclose(oracle.tolerance(c), 1e-2 + 2e-3 * np.abs(c), rtol=0, atol=0)
    rel = (oracle.tolerance(np.array([1e6]), "bf16")[0] - 1e-2) / 1e6
    assert abs(rel - (2e-3 - 2.0 ** -11 + 2.0 ** -8)) < 1e-12
    # half a bfloat16 ulp at the bottom of a binade fits under the bf16 bound
    # and not under the fp16 one
    x = np.array([8.0 + 2.0 ** -4])   # midpoint: half ulp = 2^-5 at |C| ~ 8
    assert 2.0 ** -5 <= oracle.tolerance(x, "bf16")[0]
