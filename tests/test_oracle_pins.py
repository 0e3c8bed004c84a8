"""The fp64 oracle against its pins (CPU only)."""
import pytest

import os, sys
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins as P  # noqa: E402


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_mod):
    pin(forward=oracle_mod.forward, wy_vectors=oracle_mod.wy_vectors,
        u_vectors=oracle_mod.u_vectors)


def test_oracle_thread_count_reported(oracle_mod):
    import numpy as np
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 5, 3, 4))
    v = rng.standard_normal((2, 5, 3, 4))
    be = rng.uniform(size=(2, 5, 3))
    _, _, nt = oracle_mod.forward(q, q, v, None, be, return_threads=True, n_threads=4)
    assert nt == 4
    _, _, nt = oracle_mod.forward(q, q, v, None, be, return_threads=True, n_threads=64)
    assert nt == 6  # capped at the number of (sequence, head) units
