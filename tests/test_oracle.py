"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_oracle_rejects_bad_arguments(oracle_lib):
    import numpy as np
    import oracle
    a = np.zeros((2, 3), dtype=np.uint16)
    b = np.zeros((4, 2), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(a, b, "f16", lib=oracle_lib)
    with pytest.raises(TypeError):
        oracle.gemm(a.astype(np.uint32), b[:3].astype(np.uint32), "f16", lib=oracle_lib)
    with pytest.raises(RuntimeError):
        oracle.gemm_sampled(a, b[:3], "f16", [5], [0], lib=oracle_lib)
