"""One long causal sequence through the forward: B=1, T=32768, 16 query and 8 key/value heads, d=128.

The longest prefill rows see 32768 keys, four times the 1.7B-like layer's, so the running maxima, the
lse and the fp16 range scales meet their largest row sums here.  Rows are sampled (first rows, tile
edges, the middle and the last rows, plus a uniform draw) and the oracle computes each one exactly
(the output equation of the gist.science technical summary, section "Core mechanism").
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.util import ensure_built, host, sampled_rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
T_LONG = 32768


@pytest.fixture(scope="module")
def plx():
    ensure_built()
    import softmax_learned_covariance_amd as m
    return m


def _rows(T, seed, n_uniform=24):
    r = np.random.default_rng(seed)
    uniform = np.sort(r.choice(T, size=n_uniform, replace=False))
    special = [0, 1, 31, 32, 63, 64, 8191, 8192, T // 2, T - 33, T - 32, T - 2, T - 1]
    return uniform, np.unique(np.concatenate([uniform, special]))


def test_long_context_forward_sampled(plx):
    w = W.scaled(W.WORKLOADS["layer17"], batch=1, seqlen_q=T_LONG, seqlen_k=T_LONG, seed=7)
    print(f"[long] forward B=1 T={T_LONG} Hq=16 Hkv=8 d=128 causal seed=7", flush=True)
    q, k, v, P = W.make_inputs(w, device="cuda")
    out, lse, kbar, o = plx.parallax_attn_fwd(q, k, v, P)
    torch.cuda.synchronize()
    uniform, rows = _rows(T_LONG, 29)
    ref, ref_lse, ref_kbar, ref_o = oracle.fwd(host(q), host(k), host(v), host(P), causal=True, rows=rows)
    for what, got_t, want in (("out", out, ref), ("kbar", kbar, ref_kbar), ("o", o, ref_o)):
        got = host(got_t)
        assert np.all(np.isfinite(got[:, rows])), what
        e = sampled_rel_err(got[:, rows], want[:, rows], want[:, uniform])
        print(f"[long] {what}: {e:.2e}", flush=True)
        assert e <= BF16_TOL, (what, e)
    assert np.max(np.abs(host(lse)[:, :, rows] - ref_lse[:, :, rows])) <= 1e-3
