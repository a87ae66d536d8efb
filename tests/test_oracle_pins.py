"""The oracle against its pins (CPU only).  See tests/pins.py for what pins what."""
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_float32_timing_mode():
    """The float32 mode (used only to time the oracle on the host) computes in float32 and agrees with the
    float64 default to float32 rounding; leaving the block restores float64."""
    import numpy as np
    rng = np.random.default_rng(0)
    B, T, Hq, Hkv, d = 1, 40, 2, 1, 16
    q, k, v = (rng.standard_normal(s) for s in ((B, T, Hq, d), (B, T, Hkv, d), (B, T, Hkv, d)))
    P = rng.standard_normal((Hq, d, d)) * 0.1
    dout = rng.standard_normal((B, T, Hq, d))
    ref = oracle.fwd(q, k, v, P) + oracle.bwd(q, k, v, P, dout)
    with oracle.precision(np.float32):
        got = oracle.fwd(q, k, v, P) + oracle.bwd(q, k, v, P, dout)
    assert all(g.dtype == np.float32 for g in got)
    for g, r in zip(got, ref):
        assert np.max(np.abs(g - r)) <= 1e-4 * max(1.0, np.max(np.abs(r)))
    assert oracle.fwd(q, k, v, P)[0].dtype == np.float64
