"""Head dim 64 on its own kernels (the operands staged at 64, four k-steps over d and two 32-wide output
tiles): forward and backward of the projector form against the oracle, across masks, group sizes and
splits, and the 0.6B training shape at full size on sampled heads.

Tolerance metric as in test_gpu_parity: max |gpu - oracle| / sqrt(mean(oracle^2)) per tensor, 2e-2 for bf16
inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.util import ensure_built, host, rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module")
def plx():
    ensure_built()
    import softmax_learned_covariance_amd as m
    return m


def _announce(msg):
    print(f"[d64] {msg}", flush=True)


@pytest.mark.parametrize("T,Tk,causal,window,Hkv,split", [
    (520, 520, True, 0, 8, -1),      # the 0.6B layer's grouping (2 query heads per kv head)
    (300, 300, True, 100, 8, -1),    # sliding window
    (260, 260, False, 0, 8, -1),     # bidirectional
    (129, 257, False, 64, 8, -1),    # bidirectional window, more keys than queries
    (333, 200, True, 0, 8, -1),      # causal, more queries than keys
    (257, 257, True, 0, 16, -1),     # one query head per kv head
    (257, 257, True, 0, 4, -1),      # four query heads per kv head
    (300, 300, True, 0, 2, 0),       # eight query heads per kv head, smallest split
])
def test_forward_backward_head_dim_64(plx, T, Tk, causal, window, Hkv, split):
    w = W.scaled(W.WORKLOADS["train06"], batch=2, seqlen_q=T, seqlen_k=Tk, heads_kv=Hkv, head_dim=64)
    _announce(f"d=64 forward + backward T={T} Tk={Tk} causal={causal} window={window} Hkv={Hkv} split={split}")
    q, k, v, P, dout = W.make_inputs(w, device="cuda", with_dout=True)
    kw = dict(causal=causal, window=window, split_rows=split)
    out, lse, kbar, o = plx.parallax_attn_fwd(q, k, v, P, **kw)
    grads = plx.parallax_attn_bwd(q, k, v, P, out, dout, lse, kbar, o, **kw)
    torch.cuda.synchronize()
    rf = oracle.fwd(host(q), host(k), host(v), host(P), causal=causal, window=window)
    for name, got, want in (("out", out, rf[0]), ("kbar", kbar, rf[2]), ("o", o, rf[3])):
        e = rel_err(host(got), want)
        assert e <= BF16_TOL, f"{name}: {e:.2e}"
    # rows that see no key (more queries than keys, causal) have lse = -inf on both sides
    lg, lr = host(lse), rf[1]
    fin = np.isfinite(lr)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.max(np.abs(lg[fin] - lr[fin])) <= 1e-3
    rb = oracle.bwd(host(q), host(k), host(v), host(P), host(dout), causal=causal, window=window)
    for name, got, want in zip(("dq", "dk", "dv", "dP"), grads, rb):
        e = rel_err(host(got), want)
        assert e <= BF16_TOL, f"{name}: {e:.2e}"


def test_full_size_train_step_head_dim_64(plx):
    """The 0.6B training shape (B=8, T=4096) at head dim 64, forward + backward.  Batch 0, query heads 0-1
    (all of kv head 0) exactly: dq, dk, dv; dP for heads 0-1 summed over every batch entry."""
    w = W.scaled(W.WORKLOADS["train06"], head_dim=64)
    _announce("full-size train06 at d=64, forward + backward (batch 0 / head group 0 exact)")
    q, k, v, P, dout = W.make_inputs(w, device="cuda", with_dout=True)
    out, lse, kbar, o = plx.parallax_attn_fwd(q, k, v, P)
    dq, dk, dv, dP = plx.parallax_attn_bwd(q, k, v, P, out, dout, lse, kbar, o)
    torch.cuda.synchronize()
    sl = (slice(0, 1), slice(None), slice(0, 2))
    rdq, rdk, rdv, rdP = oracle.bwd(host(q[sl]), host(k[0:1, :, 0:1]), host(v[0:1, :, 0:1]),
                                    host(P[0:2]), host(dout[sl]), causal=True)
    for name, got, want in (("dq", dq[sl], rdq), ("dk", dk[0:1, :, 0:1], rdk), ("dv", dv[0:1, :, 0:1], rdv)):
        e = rel_err(host(got), want)
        print(f"[d64] train06 {name}: {e:.2e}", flush=True)
        assert e <= BF16_TOL, (name, e)
    total = rdP.copy()
    for b in range(1, w.batch):
        total += oracle.bwd(host(q[b:b + 1, :, 0:2]), host(k[b:b + 1, :, 0:1]), host(v[b:b + 1, :, 0:1]),
                            host(P[0:2]), host(dout[b:b + 1, :, 0:2]), causal=True)[3]
    e = rel_err(host(dP[0:2]), total)
    print(f"[d64] train06 dP: {e:.2e}", flush=True)
    assert e <= BF16_TOL, e
