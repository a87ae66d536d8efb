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


def test_rows_without_keys():
    """Causal with more query rows than keys (bottom-right aligned): whole row blocks see no key.  Those
    rows give zero output and gradients and lse = -inf (all-zero weights); the others equal the same
    operator on the last Tk query rows alone, where the mask is the plain causal one."""
    import numpy as np
    rng = np.random.default_rng(1)
    B, Tq, Tk, Hq, Hkv, d = 1, 300, 40, 2, 1, 8
    q = rng.standard_normal((B, Tq, Hq, d))
    k, v = rng.standard_normal((B, Tk, Hkv, d)), rng.standard_normal((B, Tk, Hkv, d))
    P = rng.standard_normal((Hq, d, d)) * 0.1
    dout = rng.standard_normal((B, Tq, Hq, d))
    out, lse, kbar, o = oracle.fwd(q, k, v, P, causal=True)
    dq, dk, dv, dP = oracle.bwd(q, k, v, P, dout, causal=True)
    e = Tq - Tk
    assert np.all(out[:, :e] == 0) and np.all(o[:, :e] == 0) and np.all(dq[:, :e] == 0)
    assert np.all(np.isneginf(lse[:, :, :e]))
    tail = oracle.fwd(q[:, e:], k, v, P, causal=True)
    gtail = oracle.bwd(q[:, e:], k, v, P, dout[:, e:], causal=True)
    for got, want in ((out[:, e:], tail[0]), (lse[:, :, e:], tail[1]), (dq[:, e:], gtail[0]), (dk, gtail[1]),
                      (dv, gtail[2]), (dP, gtail[3])):
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
