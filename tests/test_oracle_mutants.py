"""Planted mistakes in copies of the oracle must each fail at least one pin (CPU only).

Each mutant is the oracle's source with one plausible mistake written in
(a dropped term, a flipped sign, a transposed operand, an off-by-one mask);
the real oracle module is never modified.
"""
import os
import types

import pytest

from tests import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "parallax_oracle.py")

MUTANTS = [
    ("correction sign", "out[b, rr, h] = o + c", "out[b, rr, h] = o - c"),
    ("projector transposed", "u = x @ P[h]  ", "u = x @ P[h].T"),
    # Centring one side of the covariance is enough (sum_j p_j (v_j - o) = 0), so only
    # dropping both centrings is a mistake; dropping one alone is an equivalent program.
    ("both centrings dropped",
     "t = u @ Kj.T - np.sum(u * kb, axis=1, keepdims=True)\n                w = p * t\n"
     "                c = w @ Vj - np.sum(w, axis=1, keepdims=True) * o",
     "t = u @ Kj.T\n                w = p * t\n                c = w @ Vj"),
    ("probe uses q only", "x = Qr - kb\n                if per_query", "x = Qr\n                if per_query"),
    ("key mean from values", "kb = p @ Kj\n                x = Qr", "kb = p @ Vj\n                x = Qr"),
    ("softmax scale", "scale = 1.0 / np.sqrt(d)\n    out =", "scale = 1.0 / d\n    out ="),
    ("causal off by one", "m &= j <= i\n", "m &= j < i + 0 * i\n"),
    ("causal range off by one", "hi = min(Tk, i + off + 1) if causal else Tk", "hi = min(Tk, i + off + 2) if causal else Tk"),
    ("window off by one", "m &= j > i - window", "m &= j >= i - window"),
    ("gqa mapping", "g = h // grp\n", "g = h % Hkv\n"),
    ("lse drops max", "mx[:, 0] + np.log(", "0.0 * mx[:, 0] + np.log("),
    ("bwd dkbar sign", "dkb = -go * u - Pdu", "dkb = -go * u + Pdu"),
    ("bwd P du transposed", "Pdu = du @ Ph.T", "Pdu = du @ Ph"),
    ("bwd dP transposed", "dP[h] += x.T @ du", "dP[h] += du.T @ x"),
    ("bwd dv drops 1-alpha", "dv[b, lo:hi, gk] += (p * (t + 1.0 - alpha)).T @ G", "dv[b, lo:hi, gk] += (p * t).T @ G"),
    ("bwd softmax jacobian", "ds = p * (dp - delta)", "ds = p * dp"),
    ("bwd dq scale", "dq[b, rr, h] += Pdu + scale * (ds @ Kj)", "dq[b, rr, h] += Pdu + (ds @ Kj)"),
    ("bwd dk kbar term", "+ p.T @ dkb +", "+ 0.0 * p.T @ dkb +"),
    ("decode ignores seqlens", "L = Lmax if seqlens is None else int(seqlens[b])", "L = Lmax"),
    ("probe correction sign", "out[b, rr, h] = o - (w @ Vj", "out[b, rr, h] = o + (w @ Vj"),
    ("probe centrings dropped",
     "t = Rr @ Kj.T - np.sum(Rr * kb, axis=1, keepdims=True)      # rho_i . (k_j - kbar_i)\n"
     "                w = p * t\n                out[b, rr, h] = o - (w @ Vj - np.sum(w, axis=1, keepdims=True) * o)",
     "t = Rr @ Kj.T\n                w = p * t\n                out[b, rr, h] = o - (w @ Vj)"),
    ("probe dotted with q", "t = Rr @ Kj.T", "t = Qr @ Kj.T"),
    ("paged decode page offset", "Kb = k_pages[pages_of_j, j % page]", "Kb = k_pages[pages_of_j, (j + 1) % page]"),
    ("paged decode ignores window", "lo = max(0, L - window) if window > 0 else 0\n        if L - lo == 0",
     "lo = 0\n        if L - lo == 0"),
    ("probe bwd drho sign", "drho[b, rr, h] = go * kb - (p * gv) @ Kj", "drho[b, rr, h] = (p * gv) @ Kj - go * kb"),
    ("probe bwd dp misses a(p)", "dp = gv * (1.0 + a - r) + go * r", "dp = gv * (1.0 + a - r)"),
    ("probe bwd dk rho term sign", "(p * (go - gv)).T @ Rr", "(p * (gv - go)).T @ Rr"),
    ("probe bwd dv drops a", "dv[b, lo:hi, gk] += (p * (1.0 + a - r)).T @ G", "dv[b, lo:hi, gk] += (p * (1.0 - r)).T @ G"),
    ("probe bwd dq scale", "dq[b, rr, h] = scale * (ds @ Kj)", "dq[b, rr, h] = ds @ Kj"),
    # (the key mean inside t may be any per-row constant, since sum_j p_j (v_j - o) = 0: replacing it is
    # an equivalent program, not a mistake)
]


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError, np_errors()) as e:  # noqa: F841
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake '{name}'"


def np_errors():
    import numpy as np
    return np.linalg.LinAlgError
