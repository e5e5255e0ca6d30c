"""The fp64 oracle against closed forms, finite differences and an independent
dense reference (CPU only)."""
import numpy as np
import pytest

import oracle as O
from pins import ALL_PINS


@pytest.mark.parametrize("name", list(ALL_PINS))
def test_pin(name):
    fn, tol = ALL_PINS[name]
    err = fn(O.load(), np.random.default_rng(1234))
    assert err <= tol, f"{name}: worst relative error {err:.3e} > {tol:.1e}"
