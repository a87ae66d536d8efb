"""The forward's operand roundings, emulated on the CPU (no GPU, no HIP code).

The forward kernel computes out = o + c - rs o in two passes over the key tiles (gist.science technical
summary, "Hardware-aware algorithm"; the correction of "Core mechanism"), with every operand it computes
rounded to fp16 before an MFMA: p~ = exp2(s - m + 7) for o and kbar, x = q - kbar (always as an fp16
hi + lo pair) for u = P^T x, U-hat for R = U-hat . k and alpha = U-hat . kbar, and W = p (R - alpha) for
c = sum W v and rs = sum W.  The first query rows (16 at least, 256 by default) carry p~, U-hat and W as
hi + lo pairs too.  These tests replay that arithmetic in float64 with the kernel's roundings, power-of-two
range scales and lazy running maximum written out, on a causal train06-shaped head pair (T = 256, head
dim 128, P with standard deviation 0.02), and check it against the oracle.  They pin the precision design,
not the kernel: the error concentrates in the first causal rows (they see a handful of keys, so their
outputs are many times the tensor's rms); single fp16 operands there stay well inside the 2e-2 bar, hi + lo
pairs reach fp32 level, and single bf16 operands (8 significant bits instead of 11) exceed the bar on every
seed (2.3e-2 to 3.3e-2), which is why the kernel does not use them.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

TILE, TAU, LIFT = 64, 8.0, 7.0
BAR = 2e-2


def _f16(x):
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _range_exp(m):
    """e with m 2^e in [2^14, 2^15): the power of two that scales an operand's largest entry into fp16."""
    m = np.float32(m)
    if not (m > 0) or not np.isfinite(m):
        return 0
    return 15 - int(np.frexp(m)[1])


def _operand(x, rnd, pair):
    hi = rnd(x)
    return hi + rnd(x - hi) if pair else hi


def _emulate(q, K, V, P, scale, rnd, split_rows):
    """One causal (batch, query head): q [T, d]; K, V [T, d] (bf16 values, exact in fp16); P [d, d]."""
    T, d = q.shape
    S = _f32(q @ K.T) * (scale * np.log2(np.e))              # fp32 scores, log2 units
    knorm = np.maximum.accumulate(np.linalg.norm(K, axis=1))  # largest key norm a row sees
    out = np.zeros((T, d))
    for i in range(T):
        n, pair = i + 1, i < split_rows
        # pass 1: lazy running maximum per key tile, p~ rounded, l summed from the rounded p~
        m, l, aO, aK = -np.inf, 0.0, np.zeros(d), np.zeros(d)
        for t0 in range(0, n, TILE):
            s = S[i, t0:min(n, t0 + TILE)]
            if s.max() > m + TAU:
                f = 0.0 if m == -np.inf else 2.0 ** (m - s.max())
                l, aO, aK, m = l * f, aO * f, aK * f, s.max()
            pt = _operand(_f32(np.exp2(s - m + LIFT)), rnd, pair)
            l += pt.sum()
            aO += pt @ V[t0:t0 + len(s)]
            aK += pt @ K[t0:t0 + len(s)]
        o, kb = aO / l, aK / l
        # probe: x = q - kbar as a hi + lo pair on every row, U-hat after its own range scale
        x = _f32(q[i] - kb)
        sx = 2.0 ** _range_exp(np.abs(x).max())
        u = _f32(P.T @ (_operand(x * sx, rnd, True) / sx))
        su = 2.0 ** _range_exp(np.abs(u).max())
        uh = _operand(u * su, rnd, pair) / su
        alpha = _f32(uh @ kb)
        # pass 2: W = p (R - alpha), scaled by the row's bound |U-hat| (max |k| + |kbar|) before rounding
        R = _f32(K[:n] @ uh)
        e = _range_exp(np.linalg.norm(uh) * (knorm[i] + np.linalg.norm(kb)))
        lse2 = m + np.log2(l) - LIFT
        Wt = _operand(_f32(_f32(np.exp2(S[i, :n] - lse2 + e)) * (R - alpha)), rnd, pair)
        out[i] = o + (Wt @ V[:n] - Wt.sum() * o) * 2.0 ** -e
    return out


def _workload():
    """A causal train06-shaped head pair (one sequence of 256, two query heads on one key/value head)."""
    return W.scaled(W.WORKLOADS["train06"], batch=1, seqlen_q=256, seqlen_k=256, heads_q=2, heads_kv=1)


def _inputs(seed):
    return W.make_inputs(_workload(), seed=seed)


def _emulate_heads(q, k, v, P, rnd, split_rows):
    """Emulated out [T, Hq, d] of the sequence in float64 arrays q [1, T, Hq, d], k, v [1, T, 1, d]."""
    return np.stack([_emulate(q[0, :, h], k[0, :, 0], v[0, :, 0], P[h], q.shape[-1] ** -0.5, rnd, split_rows)
                     for h in range(q.shape[2])], axis=1)


def _row_errors(seed, rnd, split_rows):
    """Per-row max |emulated - oracle| / rms(oracle out) over both heads."""
    q, k, v, P = (t.to(torch.float64).numpy() for t in _inputs(seed))
    ref = oracle.fwd(q, k, v, P, causal=True)[0][0]          # [T, Hq, d]
    got = _emulate_heads(q, k, v, P, rnd, split_rows)
    return np.abs(got - ref).max(axis=(1, 2)) / np.sqrt(np.mean(ref ** 2))


SEEDS = [0, 1, 2]


@pytest.mark.parametrize("seed", SEEDS)
def test_pairs_reach_fp32_level(seed):
    """Every row below split_rows (all 256 here, the default) on hi + lo pairs."""
    err = _row_errors(seed, _f16, split_rows=256)
    assert err.max() <= 1e-5, err.max()          # measured 1.0e-6 to 1.1e-6


@pytest.mark.parametrize("seed", SEEDS)
def test_single_fp16_operands_meet_the_bar(seed):
    """split_rows = 0: only the first 16 rows on pairs, as the kernel's floor."""
    err = _row_errors(seed, _f16, split_rows=16)
    assert err.max() <= BAR / 2, err.max()       # measured 2.2e-3 to 2.9e-3


@pytest.mark.parametrize("seed", SEEDS)
def test_single_bf16_operands_exceed_the_bar(seed):
    """The same arithmetic with bf16 operands and no pairs: the first rows carry it over the bar."""
    err = _row_errors(seed, _bf16, split_rows=0)
    assert err.max() > BAR, err.max()
    assert int(np.argmax(err)) < 32, int(np.argmax(err))
