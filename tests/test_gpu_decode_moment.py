"""The single-read decode kernel on the GPU.

One workgroup per (sequence, key/value head) reads its cache rows once and accumulates o, kbar and the
softmax-weighted moment sum_j p_j v_j k_j^T on the matrix cores; the correction is formed from them after
the last key.  It runs for one new token with bf16 inputs, head_dim 128, one or two query heads per
key/value head and at least 256 (sequence, key/value head) pairs, so the cases here are sized to that
(and the profiling hook confirms which kernel ran).  Checked against the oracle at the usual bar
(max |err| / rms <= 2e-2), against the two-pass kernels, and paged against contiguous bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.util import ensure_built, host, rel_err, sampled_rel_err, to_pages

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.fixture(scope="module")
def plx():
    ensure_built()
    import softmax_learned_covariance_amd as m
    yield m
    m.parallax_set_decode_path(m.PLX_DECODE_AUTO)


def _announce(msg):
    print(f"[moment] {msg}", flush=True)


class _Hook:
    """Records the profiling hook's events around one kernel; `ran()` tells whether it was launched in the
    last `with` block (fresh events each time: an event never recorded has no elapsed time)."""

    def __init__(self, plx, kernel):
        self.plx, self.kernel = plx, kernel
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []

    def __enter__(self):
        torch.cuda.synchronize()
        self.close()
        self.ev = [ctypes.c_void_p(), ctypes.c_void_p()]
        for e in self.ev:
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        self.plx.get_lib().parallax_set_kernel_events(self.kernel, self.ev[0], self.ev[1])
        return self

    def __exit__(self, *exc):
        self.plx.get_lib().parallax_set_kernel_events(0, None, None)

    def ran(self):
        torch.cuda.synchronize()
        ms = ctypes.c_float()
        ok = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[0], self.ev[1]) == 0
        self.hip.hipGetLastError()   # (an unrecorded event's error stays pending otherwise)
        return ok

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def _decode_ref(q, kc, vc, P, seqlens, window, scale=None):
    """Oracle decode of every sequence over its visible keys [max(0, L - window), L)."""
    B = q.shape[0]
    ref = np.zeros(q.shape)
    for b in range(B):
        L = int(seqlens[b])
        lo = max(0, L - window) if window > 0 else 0
        if L > 0:
            ref[b] = oracle.decode(host(q[b:b + 1]), host(kc[b:b + 1, lo:L]), host(vc[b:b + 1, lo:L]), host(P),
                                   scale=scale)[0]
    return ref


def _seqlens(B, L, seed):
    fixed = [L, 0, 1, 63, 64, 65, 129, L - 1]
    rng = np.random.default_rng(seed)
    rest = rng.integers(1, L + 1, size=max(0, B - len(fixed))).tolist()
    return torch.tensor((fixed + rest)[:B], dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("Hq,Hkv", [(16, 8), (8, 8)])
def test_moment_decode_matches_oracle(plx, Hq, Hkv):
    """Two and one query heads per key/value head; ragged lengths (empty, one key, tile edges, a ragged
    last tile) and windows (none, 100 keys, one key)."""
    B, L = 32, 700
    _announce(f"single-read decode Hq={Hq} Hkv={Hkv} B={B} L={L}")
    w = W.scaled(W.WORKLOADS["decode"], batch=B, seqlen_k=L, heads_q=Hq, heads_kv=Hkv)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=21 + Hkv + Hq)
    seqlens = _seqlens(B, L, seed=Hq)
    hook = _Hook(plx, plx.PLX_KERNEL_DECODE_MOMENT)
    try:
        for window in (0, 100, 1):
            with hook:
                out = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, window=window)
            assert hook.ran(), "the single-read kernel did not run"
            plx.parallax_set_decode_path(plx.PLX_DECODE_TWO_PASS)
            try:
                out2 = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, window=window)
            finally:
                plx.parallax_set_decode_path(plx.PLX_DECODE_AUTO)
            torch.cuda.synchronize()
            ref = _decode_ref(q, kc, vc, P, host(seqlens).astype(int), window)
            got = host(out)
            assert np.all(got[1] == 0), "an empty sequence gives zeros"
            err = rel_err(got, ref)
            print(f"[moment] window={window}: err {err:.2e}, vs two-pass {rel_err(got, host(out2)):.2e}", flush=True)
            assert err <= BF16_TOL, (window, err)
            assert rel_err(host(out2), ref) <= BF16_TOL
            if window == 1:   # one visible key: p = 1, the correction vanishes and out is that key's value
                for b in range(B):
                    Lb = int(seqlens[b])
                    if Lb > 0:
                        want = host(vc[b, Lb - 1]).repeat(Hq // Hkv, axis=0)
                        assert np.max(np.abs(got[b] - want)) <= 1e-5 * max(1.0, np.max(np.abs(want))), b
    finally:
        hook.close()


def test_moment_decode_moving_maximum(plx):
    """Scores that grow along the sequence (key norms rising 1x -> 6x, a softmax scale of 3/sqrt(d)), so
    the running maximum moves many times and the accumulators are rescaled; and a sequence whose largest
    score is its first key."""
    B, L, Hq, Hkv = 32, 1300, 16, 8
    _announce("single-read decode with a moving running maximum")
    w = W.scaled(W.WORKLOADS["decode"], batch=B, seqlen_k=L, heads_q=Hq, heads_kv=Hkv)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=5)
    ramp = torch.linspace(1.0, 6.0, L, device="cuda")[None, :, None, None]
    kc = (kc.float() * ramp).to(torch.bfloat16)
    kc[1] = kc[1].flip(0)
    scale = 3.0 / np.sqrt(128)
    seqlens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = plx.parallax_attn_decode(q, kc, vc, P, scale=scale)
    torch.cuda.synchronize()
    ref = _decode_ref(q, kc, vc, P, host(seqlens).astype(int), 0, scale=scale)
    err = rel_err(host(out), ref)
    print(f"[moment] moving maximum: err {err:.2e}", flush=True)
    assert err <= BF16_TOL


@pytest.mark.parametrize("page", [64, 128])
def test_moment_decode_paged(plx, page):
    """Paged caches with pages of 64 keys or more take the same kernel: bit-identical to the contiguous
    decode of the same keys, with ragged lengths and a window."""
    B, L, Hq, Hkv = 32, 900, 16, 8
    _announce(f"single-read paged decode page={page}")
    w = W.scaled(W.WORKLOADS["decode"], batch=B, seqlen_k=L, heads_q=Hq, heads_kv=Hkv)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=page)
    kp, vp, table = to_pages(kc, vc, page, seed=page)
    seqlens = _seqlens(B, L, seed=page)
    hook = _Hook(plx, plx.PLX_KERNEL_DECODE_MOMENT)
    try:
        for window in (0, 333):
            ref_c = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, window=window)
            with hook:
                out = plx.parallax_attn_decode_paged(q, kp, vp, table, P, seqlens=seqlens, seqlen_k=L, window=window)
            assert hook.ran(), "the single-read kernel did not run"
            torch.cuda.synchronize()
            assert torch.equal(out, ref_c), window
            ref = _decode_ref(q, kc, vc, P, host(seqlens).astype(int), window)
            assert rel_err(host(out), ref) <= BF16_TOL
    finally:
        hook.close()


def test_moment_decode_outputs(plx):
    """bf16 out is the fp32 out rounded; the correction ratio |out - o| / |out| against the oracle's."""
    B, L, Hq, Hkv = 32, 800, 16, 8
    _announce("single-read decode: bf16 out, correction ratio")
    w = W.scaled(W.WORKLOADS["decode"], batch=B, seqlen_k=L, heads_q=Hq, heads_kv=Hkv)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=77)
    seqlens = _seqlens(B, L, seed=3)
    out32, cor = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, cor=True)
    out16 = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out16, out32.to(torch.bfloat16))
    sl = host(seqlens).astype(int)
    ref = _decode_ref(q, kc, vc, P, sl, 0)
    ref0 = _decode_ref(q, kc, vc, torch.zeros_like(P), sl, 0)
    num = np.linalg.norm(ref - ref0, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    want = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    assert np.all(host(cor)[1] == 0)
    assert rel_err(host(cor), want) <= BF16_TOL


def test_full_size_decode_moment_vs_two_pass(plx):
    """64 sequences of 32768 keys, 16 query and 8 key/value heads: the single-read kernel against the
    two-pass kernels on every output, and against the oracle on sampled sequences."""
    w = W.WORKLOADS["decode"]
    _announce("full-size decode: single-read vs two-pass")
    q, kc, vc, P = W.make_inputs(w, device="cuda")
    hook = _Hook(plx, plx.PLX_KERNEL_DECODE_MOMENT)
    try:
        with hook:
            out = plx.parallax_attn_decode(q, kc, vc, P)
        assert hook.ran(), "the single-read kernel did not run"
    finally:
        hook.close()
    plx.parallax_set_decode_path(plx.PLX_DECODE_TWO_PASS)
    try:
        out2 = plx.parallax_attn_decode(q, kc, vc, P)
    finally:
        plx.parallax_set_decode_path(plx.PLX_DECODE_AUTO)
    torch.cuda.synchronize()
    d = rel_err(host(out), host(out2))
    print(f"[moment] full size: single-read vs two-pass {d:.2e}", flush=True)
    assert d <= BF16_TOL
    bsel = [0, 37, 63]
    ref = oracle.decode(host(q[bsel]), host(kc[bsel]), host(vc[bsel]), host(P))
    err = sampled_rel_err(host(out)[bsel], ref, ref)
    print(f"[moment] full size sampled vs oracle {err:.2e}", flush=True)
    assert err <= BF16_TOL


def _pow2(x, e):
    """x * 2^e exactly (bf16 keeps its significand; the exponents used here stay in range)."""
    return (x.float() * (2.0 ** e)).to(x.dtype)


@pytest.mark.parametrize("c", [20, -20])
def test_moment_decode_value_scale_is_exact(plx, c):
    """out is linear in V and the kernel's value scale is a power of two set from the data: V * 2^c gives
    out * 2^c bit for bit."""
    _announce(f"single-read decode: V * 2^{c}")
    w = W.scaled(W.WORKLOADS["decode"], batch=32, seqlen_k=400, heads_q=16, heads_kv=8)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=11)
    seqlens = _seqlens(32, 400, seed=2)
    hook = _Hook(plx, plx.PLX_KERNEL_DECODE_MOMENT)
    try:
        with hook:
            out = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens)
        assert hook.ran(), "the single-read kernel did not run"
    finally:
        hook.close()
    outs = plx.parallax_attn_decode(q, kc, _pow2(vc, c), P, seqlens=seqlens)
    torch.cuda.synchronize()
    assert torch.equal(outs, out * 2.0 ** c)


@pytest.mark.parametrize("a", [10, -10])
def test_moment_decode_score_preserving_scale_is_exact(plx, a):
    """(q, k, P, softmax scale) -> (2^a q, 2^a k, 2^-2a P, 2^-2a scale) leaves every score and the output
    unchanged; the key scale follows k, so the output is the same bit for bit."""
    _announce(f"single-read decode: (q, k, P, scale) * (2^{a}, 2^{a}, 2^{-2 * a}, 2^{-2 * a})")
    w = W.scaled(W.WORKLOADS["decode"], batch=32, seqlen_k=400, heads_q=16, heads_kv=8)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=12)
    seqlens = _seqlens(32, 400, seed=3)
    scale = 128 ** -0.5
    out = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, scale=scale)
    outs = plx.parallax_attn_decode(_pow2(q, a), _pow2(kc, a), vc, _pow2(P, -2 * a), seqlens=seqlens,
                                    scale=scale * 2.0 ** (-2 * a))
    torch.cuda.synchronize()
    assert torch.equal(outs, out)


@pytest.mark.parametrize("which,e,Hq", [("V", 12, 16), ("V", 20, 16), ("K", 6, 16), ("K", 12, 16), ("K", 20, 16),
                                         ("K", 12, 8)])
def test_moment_decode_outlier_rows(plx, which, e, Hq):
    """The last two keys of every sequence 2^e larger than the rest (values or keys): the value scale then
    puts the other values 2^e lower in fp16 (still in its normal range), and a key tile's scale follows its
    largest key; against the oracle at the usual bar.

    Keys 2^12 and more larger dominate their softmax, so kbar is close to them and the moment form's
    M u / l and alpha o are each far larger than their difference; the kernel detects that and forms
    those heads' corrections directly from a second read of their keys."""
    _announce(f"single-read decode: outlier {which} rows * 2^{e}, {Hq} query heads")
    B, L = 32, 500
    w = W.scaled(W.WORKLOADS["decode"], batch=B, seqlen_k=L, heads_q=Hq, heads_kv=8)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=13)
    t = (vc if which == "V" else kc).clone()
    t[:, L - 2:] = _pow2(t[:, L - 2:], e)
    if which == "V":
        vc = t
    else:
        kc = t
    hook = _Hook(plx, plx.PLX_KERNEL_DECODE_MOMENT)
    try:
        with hook:
            out = plx.parallax_attn_decode(q, kc, vc, P)
        assert hook.ran(), "the single-read kernel did not run"
    finally:
        hook.close()
    torch.cuda.synchronize()
    ref = _decode_ref(q, kc, vc, P, [L] * B, 0)
    err = rel_err(host(out), ref)
    print(f"[moment] outlier {which} 2^{e} Hq={Hq}: err {err:.2e}", flush=True)
    assert err <= BF16_TOL


def test_moment_decode_direct_correction_paged(plx):
    """The direct correction (key rows 2^12 larger: the heads they dominate take it) reads its keys through
    the page table too: bit-identical to the contiguous decode, with ragged lengths and a window.  Against
    the oracle the worst head is one that the outliers do not dominate but push near fp32's limit
    (1.8e-2 here; the two-pass kernels give 2.4e-2 on it)."""
    B, L, Hq, Hkv = 32, 700, 16, 8
    _announce("single-read decode: direct correction through a paged cache")
    w = W.scaled(W.WORKLOADS["decode"], batch=B, seqlen_k=L, heads_q=Hq, heads_kv=Hkv)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=14)
    kc = kc.clone()
    kc[:, 200:202] = _pow2(kc[:, 200:202], 12)
    kp, vp, table = to_pages(kc, vc, 64, seed=5)
    seqlens = _seqlens(B, L, seed=6)
    hook = _Hook(plx, plx.PLX_KERNEL_DECODE_MOMENT)
    try:
        for window in (0, 600):
            ref_c = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, window=window)
            with hook:
                out = plx.parallax_attn_decode_paged(q, kp, vp, table, P, seqlens=seqlens, seqlen_k=L, window=window)
            assert hook.ran(), "the single-read kernel did not run"
            torch.cuda.synchronize()
            assert torch.equal(out, ref_c), window
            ref = _decode_ref(q, kc, vc, P, host(seqlens).astype(int), window)
            err = rel_err(host(out), ref)
            print(f"[moment] direct correction paged window={window}: err {err:.2e}", flush=True)
            assert err <= BF16_TOL
    finally:
        hook.close()


def test_moment_decode_selection(plx):
    """Below 256 (sequence, key/value head) pairs, with more than two query heads per key/value head, with
    several new tokens or with pages under 64 keys the two-pass kernels run instead."""
    _announce("single-read decode: where it applies")
    w = W.scaled(W.WORKLOADS["decode"], batch=32, seqlen_k=300, heads_q=16, heads_kv=8)
    q, kc, vc, P = W.make_inputs(w, device="cuda", seed=8)
    hook = _Hook(plx, plx.PLX_KERNEL_DECODE_MOMENT)
    try:
        cases = [("32 x 8 pairs", True, lambda: plx.parallax_attn_decode(q, kc, vc, P)),
                 ("16 x 8 pairs", False, lambda: plx.parallax_attn_decode(q[:16], kc[:16], vc[:16], P))]
        q4 = q.reshape(32, 1, 16, 128).expand(32, 2, 16, 128).contiguous()
        cases.append(("two tokens", False, lambda: plx.parallax_attn_decode(q4, kc, vc, P)))
        kp, vp, table = to_pages(kc, vc, 32, seed=4)
        cases.append(("32-key pages", False, lambda: plx.parallax_attn_decode_paged(q, kp, vp, table, P, seqlen_k=300)))
        for name, want, call in cases:
            with hook:
                call()
            assert hook.ran() == want, name
        plx.parallax_set_decode_path(plx.PLX_DECODE_TWO_PASS)
        try:
            with hook:
                plx.parallax_attn_decode(q, kc, vc, P)
            assert not hook.ran(), "two-pass forced"
        finally:
            plx.parallax_set_decode_path(plx.PLX_DECODE_AUTO)
    finally:
        hook.close()
