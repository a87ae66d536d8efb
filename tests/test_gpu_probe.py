"""GPU parity of the probe-form forward (caller-supplied rho per query row) against oracle.fwd_probe.

Same metric and bars as the other parity tests: max |gpu - oracle| / rms(oracle) <= 2e-2 for bf16
inputs, log-sum-exp within 1e-3.  rho is drawn by workloads.make_probe.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.util import ensure_built, host, rel_err, sampled_rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module")
def plx():
    ensure_built()
    import softmax_learned_covariance_amd as m
    return m


def _announce(msg):
    print(f"[probe] {msg}", flush=True)


def _run(plx, q, k, v, rho, **kw):
    out = plx.parallax_attn_fwd_probe(q, k, v, rho, **kw)
    torch.cuda.synchronize()
    return out


def _check(plx, w, causal=True, window=0, split=-1, rho_gain=1.0):
    q, k, v, _ = W.make_inputs(w, device="cuda")
    rho = W.make_probe(w, device="cuda")
    if rho_gain != 1.0:
        rho = (rho.float() * rho_gain).to(rho.dtype)
    out, lse = _run(plx, q, k, v, rho, causal=causal, window=window, split_rows=split)[:2]
    ref, ref_lse = oracle.fwd_probe(host(q), host(k), host(v), host(rho), causal=causal, window=window)[:2]
    e = rel_err(host(out), ref)
    assert e <= BF16_TOL, e
    got_lse = host(lse)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.max(np.abs(got_lse[fin] - ref_lse[fin]), initial=0.0) <= 1e-3
    return e


@pytest.mark.parametrize("T,Tk,causal,window,Hkv,split", [
    (1000, 1000, True, 0, 8, -1),    # several row blocks and key tiles, ragged tail
    (333, 333, True, 0, 8, -1),
    (300, 700, True, 0, 8, -1),      # more keys than queries
    (333, 200, True, 0, 8, -1),      # more queries than keys: the first rows see no key
    (700, 700, True, 100, 8, -1),    # sliding window
    (260, 260, False, 0, 8, -1),     # bidirectional
    (129, 257, False, 64, 8, -1),    # bidirectional window
    (257, 257, True, 0, 16, -1),     # one query head per key/value head
    (257, 257, True, 0, 4, -1),      # four query heads per key/value head
    (450, 450, True, 200, 2, 0),     # eight query heads per key/value head, smallest split
    (1, 1, True, 0, 8, -1),
])
def test_probe_small(plx, T, Tk, causal, window, Hkv, split):
    w = W.scaled(W.WORKLOADS["layer06"], batch=2, seqlen_q=T, seqlen_k=Tk, heads_kv=Hkv)
    _announce(f"T={T} Tk={Tk} causal={causal} window={window} Hkv={Hkv} split={split}")
    _check(plx, w, causal, window, split)


@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 200, 6, 3), (3, 5, 2, 1), (1, 97, 8, 2)])
def test_probe_odd_shapes(plx, B, T, Hq, Hkv):
    _announce(f"odd shapes B={B} T={T} Hq={Hq} Hkv={Hkv}")
    w = W.scaled(W.WORKLOADS["layer06"], batch=B, seqlen_q=T, seqlen_k=T, heads_q=Hq, heads_kv=Hkv)
    _check(plx, w)


@pytest.mark.parametrize("gain", [0.0, 20.0])
def test_probe_scale(plx, gain):
    """rho = 0 is plain softmax attention; a probe 20x larger makes the correction dominate the output."""
    _announce(f"rho gain {gain}")
    w = W.scaled(W.WORKLOADS["layer06"], batch=1, seqlen_q=600, seqlen_k=600)
    _check(plx, w, rho_gain=gain)


def test_probe_zero_matches_plain_forward(plx):
    """rho = 0 and P = 0 both reduce to softmax attention: the two entry points agree."""
    _announce("rho = 0 against the two-pass forward with P = 0")
    w = W.scaled(W.WORKLOADS["layer06"], batch=1, seqlen_q=520, seqlen_k=520)
    q, k, v, P = W.make_inputs(w, device="cuda")
    out, lse = _run(plx, q, k, v, torch.zeros_like(q))[:2]
    out2, lse2, _, o2 = plx.parallax_attn_fwd(q, k, v, torch.zeros_like(P))
    torch.cuda.synchronize()
    # each side rounds p~ to fp16 against its own running maxima (per 32 and per 64 keys): the
    # denominators agree to the fp16 rounding of their terms, not bit for bit
    assert rel_err(host(out), host(o2)) <= 1e-2
    assert np.max(np.abs(host(lse) - host(lse2))) <= 1e-3


def test_probe_empty_and_degenerate(plx):
    _announce("empty and degenerate shapes")
    bf = torch.bfloat16
    q = torch.randn((1, 5, 2, 128), device="cuda").to(bf)
    k = torch.empty((1, 0, 1, 128), device="cuda", dtype=bf)
    out, lse = _run(plx, q, k, k, q)[:2]
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    q0 = torch.empty((1, 0, 2, 128), device="cuda", dtype=bf)
    k1 = torch.randn((1, 4, 1, 128), device="cuda").to(bf)
    out = _run(plx, q0, k1, k1, q0)[0]
    assert out.numel() == 0
    qb = torch.empty((0, 4, 2, 128), device="cuda", dtype=bf)
    kb = torch.empty((0, 4, 1, 128), device="cuda", dtype=bf)
    out = _run(plx, qb, kb, kb, qb)[0]
    assert out.numel() == 0


def test_probe_determinism_and_split_floor(plx):
    _announce("determinism, split_rows 0 vs 16")
    w = W.scaled(W.WORKLOADS["layer06"], batch=1, seqlen_q=640, seqlen_k=640)
    q, k, v, _ = W.make_inputs(w, device="cuda")
    rho = W.make_probe(w, device="cuda")
    a = _run(plx, q, k, v, rho, split_rows=0)
    b = _run(plx, q, k, v, rho, split_rows=16)
    c = _run(plx, q, k, v, rho, split_rows=16)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(y, z)


def test_probe_full_size_sampled(plx):
    """The 1.7B layer at full size (B=2, T=8192): sampled rows computed one by one by the oracle."""
    w = W.WORKLOADS["layer17"]
    _announce("full-size layer17 (sampled rows)")
    q, k, v, _ = W.make_inputs(w, device="cuda")
    rho = W.make_probe(w, device="cuda")
    out, lse = _run(plx, q, k, v, rho)[:2]
    r = np.random.default_rng(23)
    T = w.seqlen_q
    uniform = np.sort(r.choice(T, size=24, replace=False))
    special = np.array([0, 1, 2, 15, 16, 63, 64, 255, 256, 257, 511, T // 2, T - 2, T - 1])
    rows = np.unique(np.concatenate([uniform, special]))
    bsel = [0, w.batch - 1]
    ref, ref_lse = oracle.fwd_probe(host(q[bsel]), host(k[bsel]), host(v[bsel]), host(rho[bsel]),
                                    causal=True, rows=rows)[:2]
    got = host(out[bsel])
    e = sampled_rel_err(got[:, rows], ref[:, rows], ref[:, uniform])
    assert e <= BF16_TOL, e
    assert np.max(np.abs(host(lse[bsel])[:, :, rows] - ref_lse[:, :, rows])) <= 1e-3


# --------------------------------------------------------------------------------------
# backward (drho and the gradients of q, k, v)
# --------------------------------------------------------------------------------------

def _check_bwd(plx, w, causal=True, window=0, split=-1):
    q, k, v, _, dout = W.make_inputs(w, device="cuda", with_dout=True)
    rho = W.make_probe(w, device="cuda")
    kw = dict(causal=causal, window=window, split_rows=split)
    out, lse, o, rk = _run(plx, q, k, v, rho, **kw)
    grads = plx.parallax_attn_bwd_probe(q, k, v, rho, out, dout, lse, o, rk, **kw)
    torch.cuda.synchronize()
    hq, hk, hv, hr = host(q), host(k), host(v), host(rho)
    _, _, ref_o, ref_rk = oracle.fwd_probe(hq, hk, hv, hr, causal=causal, window=window)
    assert rel_err(host(o), ref_o) <= BF16_TOL
    assert rel_err(host(rk), ref_rk) <= BF16_TOL
    ref = oracle.bwd_probe(hq, hk, hv, hr, host(dout), causal=causal, window=window)
    for name, got, want in zip(("dq", "dk", "dv", "drho"), grads, ref):
        e = rel_err(host(got), want)
        assert e <= BF16_TOL, f"{name}: {e:.2e}"


@pytest.mark.parametrize("T,Tk,causal,window,Hkv,split", [
    (520, 520, True, 0, 8, -1),      # more rows than the default split, ragged tail
    (300, 300, True, 100, 8, -1),    # sliding window
    (260, 260, False, 0, 8, -1),     # bidirectional
    (129, 257, False, 64, 8, -1),    # bidirectional window, more keys than queries
    (200, 333, True, 0, 8, -1),      # causal, more keys than queries
    (333, 200, True, 0, 8, -1),      # causal, more queries than keys: the first rows see no key
    (257, 257, True, 0, 16, -1),     # one query head per key/value head
    (257, 257, True, 0, 4, -1),      # four query heads per key/value head
    (300, 300, True, 0, 8, 0),       # smallest split: rows >= 16 on single fp16 operands
    (300, 300, True, 0, 2, -1),      # eight query heads per key/value head
])
def test_probe_backward_small(plx, T, Tk, causal, window, Hkv, split):
    w = W.scaled(W.WORKLOADS["train06"], batch=2, seqlen_q=T, seqlen_k=Tk, heads_kv=Hkv)
    _announce(f"backward T={T} Tk={Tk} causal={causal} window={window} Hkv={Hkv} split={split}")
    _check_bwd(plx, w, causal, window, split)


@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 200, 6, 3), (3, 5, 2, 1), (1, 97, 8, 2)])
def test_probe_backward_odd_shapes(plx, B, T, Hq, Hkv):
    _announce(f"backward odd shapes B={B} T={T} Hq={Hq} Hkv={Hkv}")
    w = W.scaled(W.WORKLOADS["train06"], batch=B, seqlen_q=T, seqlen_k=T, heads_q=Hq, heads_kv=Hkv)
    _check_bwd(plx, w)


def test_probe_backward_empty(plx):
    _announce("backward with no keys / no queries")
    bf = torch.bfloat16
    q = torch.randn((1, 5, 2, 128), device="cuda").to(bf)
    k = torch.empty((1, 0, 1, 128), device="cuda", dtype=bf)
    out, lse, o, rk = _run(plx, q, k, k, q)
    dq, dk, dv, drho = plx.parallax_attn_bwd_probe(q, k, k, q, out, q, lse, o, rk)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and torch.all(drho == 0) and dk.numel() == 0
    q0 = torch.empty((1, 0, 2, 128), device="cuda", dtype=bf)
    k1 = torch.randn((1, 4, 1, 128), device="cuda").to(bf)
    out, lse, o, rk = _run(plx, q0, k1, k1, q0)
    dq, dk, dv, drho = plx.parallax_attn_bwd_probe(q0, k1, k1, q0, out, q0, lse, o, rk)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0) and dq.numel() == 0


def test_probe_backward_determinism(plx):
    _announce("backward determinism")
    w = W.scaled(W.WORKLOADS["train06"], batch=1, seqlen_q=640, seqlen_k=640)
    q, k, v, _, dout = W.make_inputs(w, device="cuda", with_dout=True)
    rho = W.make_probe(w, device="cuda")
    f = _run(plx, q, k, v, rho)
    a = plx.parallax_attn_bwd_probe(q, k, v, rho, f[0], dout, *f[1:])
    b = plx.parallax_attn_bwd_probe(q, k, v, rho, f[0], dout, *f[1:])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_probe_full_size_train_step_sampled(plx):
    """The 0.6B training shape at full size (B=8, T=4096), probe form forward + backward.  Batch 0, query
    heads 0-1 (all of key/value head 0) are computed exactly by the oracle: dq, drho for those heads, dk, dv
    for that key/value head."""
    w = W.WORKLOADS["train06"]
    _announce("full-size train06 probe forward + backward (sampled)")
    q, k, v, _, dout = W.make_inputs(w, device="cuda", with_dout=True)
    rho = W.make_probe(w, device="cuda")
    out, lse, o, rk = _run(plx, q, k, v, rho)
    dq, dk, dv, drho = plx.parallax_attn_bwd_probe(q, k, v, rho, out, dout, lse, o, rk)
    torch.cuda.synchronize()
    sl = (slice(0, 1), slice(None), slice(0, 2))
    rdq, rdk, rdv, rdr = oracle.bwd_probe(host(q[sl]), host(k[0:1, :, 0:1]), host(v[0:1, :, 0:1]),
                                          host(rho[sl]), host(dout[sl]), causal=True)
    assert rel_err(host(dq[sl]), rdq) <= BF16_TOL
    assert rel_err(host(drho[sl]), rdr) <= BF16_TOL
    assert rel_err(host(dk[0:1, :, 0:1]), rdk) <= BF16_TOL
    assert rel_err(host(dv[0:1, :, 0:1]), rdv) <= BF16_TOL


@pytest.mark.parametrize("T,window", [(1000, 0), (333, 100)])
def test_probe_head_dim_64(plx, T, window):
    """Head dim 64 (the MFMA kernels instantiated for 64) for the probe-form forward and backward."""
    w = W.scaled(W.WORKLOADS["train06"], batch=2, seqlen_q=T, seqlen_k=T, head_dim=64)
    _announce(f"probe forward + backward d=64 T={T} window={window}")
    _check(plx, w, True, window)
    _check_bwd(plx, w, True, window)


@pytest.mark.parametrize("T,Hkv", [(1000, 8), (257, 16)])
def test_forward_head_dim_64(plx, T, Hkv):
    """The projector-form forward at head dim 64 on the MFMA path: out, o, kbar and lse against the oracle."""
    w = W.scaled(W.WORKLOADS["layer06"], batch=2, seqlen_q=T, seqlen_k=T, heads_kv=Hkv, head_dim=64)
    _announce(f"forward d=64 T={T} Hkv={Hkv}")
    q, k, v, P = W.make_inputs(w, device="cuda")
    out, lse, kbar, o = plx.parallax_attn_fwd(q, k, v, P)
    torch.cuda.synchronize()
    ref = oracle.fwd(host(q), host(k), host(v), host(P), causal=True)
    assert rel_err(host(out), ref[0]) <= BF16_TOL
    assert rel_err(host(o), ref[3]) <= BF16_TOL
    assert rel_err(host(kbar), ref[2]) <= BF16_TOL
    assert np.max(np.abs(host(lse) - ref[1])) <= 1e-3
