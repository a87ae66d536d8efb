"""Pins of the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle module (so a mutation test can run the same pins
against deliberately broken copies of it) and raises AssertionError when the
oracle disagrees.  None of them re-types the oracle's own formula: each compares
it with a library routine (torch SDPA, numpy.linalg.lstsq, numpy.cov,
scipy.special.softmax), a closed form, a hand-worked example, an invariant, or
central finite differences.

Passages (gist.science technical summary of "Parallax: Parameterized Local
Linear Attention for Language Modeling"): "Core mechanism" gives the output as
softmax attention plus the key/value covariance applied to a probe, the probe
replacing the per-query solve of exact local linear attention (which inverts
the key covariance); "Problem statement" describes LLA as the local *linear*
estimator replacing the local-constant (Nadaraya-Watson) estimator of softmax
attention.  The encorp.ai blog ("Parallax keeps softmax" and its FAQ) states
that a zero projector gives exactly softmax attention.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_case(seed, B=2, Tq=20, Tk=20, Hq=4, Hkv=2, d=6, p_std=0.3):
    r = _rng(seed)
    q = r.standard_normal((B, Tq, Hq, d))
    k = r.standard_normal((B, Tk, Hkv, d))
    v = r.standard_normal((B, Tk, Hkv, d))
    P = r.standard_normal((Hq, d, d)) * p_std
    return q, k, v, P


def _close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"
    return err


def _sdpa(q, k, v, causal, scale, Tq_full=None):
    """torch scaled_dot_product_attention in float64 on the CPU, GQA by repeating K/V heads."""
    Hq, Hkv = q.shape[2], k.shape[2]
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)
    K = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    V = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


# ---------------------------------------------------------------------------
# forward pins
# ---------------------------------------------------------------------------

def pin_zero_projector_is_sdpa(orc):
    """P = 0 gives softmax attention: compare with torch SDPA (square causal, non-causal, GQA, custom scale)."""
    q, k, v, P = _rand_case(1)
    for causal in (True, False):
        for scale in (None, 0.37):
            out, _, _, o = orc.fwd(q, k, v, np.zeros_like(P), causal=causal, scale=scale)
            ref = _sdpa(q, k, v, causal, scale if scale else 1.0 / math.sqrt(q.shape[-1]))
            _close(out, ref, 1e-12, f"P=0 vs SDPA causal={causal} scale={scale}")
            _close(o, ref, 1e-12, "softmax branch vs SDPA")


def pin_bottom_right_alignment(orc):
    """Tq < Tk causal: the queries are the last Tq positions of a square causal problem (SDPA on the square)."""
    r = _rng(2)
    B, Tk, Tq, Hq, Hkv, d = 1, 17, 5, 2, 1, 4
    qfull = r.standard_normal((B, Tk, Hq, d))
    k = r.standard_normal((B, Tk, Hkv, d))
    v = r.standard_normal((B, Tk, Hkv, d))
    P = np.zeros((Hq, d, d))
    out, _, _, _ = orc.fwd(qfull[:, -Tq:], k, v, P, causal=True)
    ref = _sdpa(qfull, k, v, True, 1.0 / math.sqrt(d))[:, -Tq:]
    _close(out, ref, 1e-12, "bottom-right causal alignment")


def pin_mask_counts(orc):
    """Q = 0 makes every visible key equally likely, so exp(lse) is the visible-key count.

    Counts from the mask's plain description: a causal query at absolute
    position i' = i + (Tk - Tq) sees keys 0..i'; a window of W keeps the W keys
    ending at the query (keys i'-W+1..i'); non-causal sees all keys.
    """
    r = _rng(3)
    for (Tq, Tk, causal, window) in [(9, 9, True, 0), (4, 11, True, 0), (9, 9, True, 3),
                                     (6, 10, True, 4), (7, 7, False, 0), (5, 8, False, 2)]:
        d = 3
        q = np.zeros((1, Tq, 1, d))
        k = r.standard_normal((1, Tk, 1, d))
        v = r.standard_normal((1, Tk, 1, d))
        _, lse, _, _ = orc.fwd(q, k, v, np.zeros((1, d, d)), causal=causal, window=window)
        got = np.rint(np.exp(lse[0, 0])).astype(int)
        want = []
        for i in range(Tq):
            ip = i + Tk - Tq
            last = min(ip, Tk - 1) if causal else Tk - 1
            first = max(0, ip - window + 1) if window > 0 else 0
            want.append(max(0, last - first + 1))
        assert list(got) == want, f"mask counts Tq={Tq} Tk={Tk} causal={causal} W={window}: {got} vs {want}"


def pin_exact_lla_is_ridge_wls(orc):
    """Per-query P = (Sigma_q + lam I)^-1 makes the output the brute-force ridge weighted least-squares intercept.

    For query i with softmax weights p_j (scipy.special.softmax of its visible
    scores), fit v_j ~ a + B (k_j - q_i) minimising sum_j p_j |v_j - a - B(k_j - q_i)|^2
    + lam |B|_F^2 (intercept unpenalised) by numpy.linalg.lstsq on the
    augmented system; the prediction at the query point is a.
    """
    r = _rng(4)
    B, T, H, d, lam = 1, 24, 1, 4, 1e-2
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d))
    v = r.standard_normal((B, T, H, d))
    scale = 1.0 / math.sqrt(d)
    Pq = orc.exact_lla_projector(q, k, causal=True, lam=lam)
    out, _, _, _ = orc.fwd(q, k, v, Pq, causal=True)
    for i in range(T):
        Kj, Vj = k[0, :i + 1, 0], v[0, :i + 1, 0]
        p = scipy.special.softmax(scale * (Kj @ q[0, i, 0]))
        sw = np.sqrt(p)[:, None]
        A = np.vstack([np.hstack([sw, sw * (Kj - q[0, i, 0])]),
                       np.hstack([np.zeros((d, 1)), math.sqrt(lam) * np.eye(d)])])
        rhs = np.vstack([sw * Vj, np.zeros((d, d))])
        theta, *_ = np.linalg.lstsq(A, rhs, rcond=None)
        _close(out[0, i, 0], theta[0], 1e-9, f"exact LLA row {i}")


def _weighted_cov(x, y, p):
    """Softmax-weighted cross-covariance sum_j p_j (x_j - xbar)(y_j - ybar)^T via numpy.cov."""
    dx = x.shape[1]
    c = np.cov(np.hstack([x, y]).T, aweights=p, bias=True)
    return c[:dx, dx:]


def pin_covariance_form(orc):
    """out_i - o_i = Sigma_KV^(i) u_i with Sigma_KV from numpy.cov, u_i = P_h^T (q_i - kbar_i).

    Run once with rank-one projectors P_h = e_b e_a^T (so u has the single
    entry u[a] = (q - kbar)[b]: this fixes P's orientation) and once with
    dense random projectors; GQA 4 query heads on 2 key/value heads.
    """
    q, k, v, _ = _rand_case(5, B=1, Tq=9, Tk=12, Hq=4, Hkv=2, d=5)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    r = _rng(6)
    Ps = []
    Pr = np.zeros((4, d, d))
    for h, (bb, aa) in enumerate([(0, 1), (3, 2), (4, 4), (1, 0)]):
        Pr[h, bb, aa] = 1.0
    Ps.append(Pr)
    Ps.append(r.standard_normal((4, d, d)) * 0.5)
    for P in Ps:
        out, _, _, _ = orc.fwd(q, k, v, P, causal=True)
        for h in range(4):
            g = h // 2
            for i in range(q.shape[1]):
                ip = i + 3
                Kj, Vj = k[0, :ip + 1, g], v[0, :ip + 1, g]
                p = scipy.special.softmax(scale * (Kj @ q[0, i, h]))
                o = np.average(Vj, axis=0, weights=p)
                kb = np.average(Kj, axis=0, weights=p)
                u = P[h].T @ (q[0, i, h] - kb)
                want = o + _weighted_cov(Vj, Kj, p) @ u
                _close(out[0, i, h], want, 1e-10, f"covariance form head {h} row {i}")


def pin_constant_values(orc):
    """Constant values: every centred value is zero, so the output is that value for any projector."""
    q, k, v, P = _rand_case(7, p_std=3.0)
    v[:] = v[:, :1]
    out, _, _, _ = orc.fwd(q, k, v, P, causal=True)
    for h in range(q.shape[2]):
        _close(out[:, :, h], np.broadcast_to(v[:, :1, h // 2], out[:, :, h].shape), 1e-12, "constant V")


def pin_single_key_rows(orc):
    """A query that sees one key returns that key's value: first causal row, and every row with window = 1."""
    q, k, v, P = _rand_case(8, p_std=2.0)
    out, _, _, _ = orc.fwd(q, k, v, P, causal=True)
    for h in range(q.shape[2]):
        _close(out[:, 0, h], v[:, 0, h // 2], 1e-12, "first causal row")
    out, _, _, _ = orc.fwd(q, k, v, P, causal=True, window=1)
    for h in range(q.shape[2]):
        _close(out[:, :, h], v[:, :, h // 2], 1e-12, "window = 1")


def pin_affine_values(orc):
    """Affine values v = A k + b with the exact-LLA projector.

    Closed form (ridge normal equations with an unpenalised intercept):
    out - (A q + b) = -lam A (Sigma_q + lam I)^-1 (q - kbar); Sigma_q and kbar
    from numpy.cov / numpy.average with scipy softmax weights.  As lam -> 0,
    rows that see at least d+1 keys reproduce A q + b exactly.
    """
    r = _rng(9)
    B, T, H, d = 1, 20, 1, 3
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d))
    A = r.standard_normal((d, d))
    bvec = r.standard_normal(d)
    v = np.einsum("btha,ca->bthc", k, A) + bvec
    scale = 1.0 / math.sqrt(d)
    for lam in (1e-2, 1e-11):
        Pq = orc.exact_lla_projector(q, k, causal=True, lam=lam)
        out, _, _, _ = orc.fwd(q, k, v, Pq, causal=True)
        for i in range(T):
            Kj = k[0, :i + 1, 0]
            p = scipy.special.softmax(scale * (Kj @ q[0, i, 0]))
            kb = np.average(Kj, axis=0, weights=p)
            cov = np.atleast_2d(np.cov(Kj.T, aweights=p, bias=True)) if i > 0 else np.zeros((d, d))
            lin = A @ q[0, i, 0] + bvec
            if lam > 1e-6:
                want = lin - lam * A @ np.linalg.solve(cov + lam * np.eye(d), q[0, i, 0] - kb)
                _close(out[0, i, 0], want, 1e-9, f"affine V closed form row {i}")
            elif i + 1 >= d + 1:
                _close(out[0, i, 0], lin, 1e-6, f"affine V reproduced row {i}")


def pin_linear_in_projector(orc):
    """The correction is linear in P: out(aP) - o = a (out(P) - o)."""
    q, k, v, P = _rand_case(10)
    out1, _, _, o = orc.fwd(q, k, v, P, causal=True)
    out2, _, _, _ = orc.fwd(q, k, v, -2.5 * P, causal=True)
    _close(out2 - o, -2.5 * (out1 - o), 1e-11, "linearity in P")


def pin_hand_examples(orc):
    """Hand-worked closed-form examples stored in tests/golden/hand_examples.json."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"])[None, :, None, :]
        k = np.array(c["k"])[None, :, None, :]
        v = np.array(c["v"])[None, :, None, :]
        P = np.array(c["P"])[None]
        out, lse, _, _ = orc.fwd(q, k, v, P, causal=c["causal"], scale=c["scale"])
        _close(out[0, :, 0], np.array(c["out"]), 1e-14, c["name"] + " out")
        _close(lse[0, 0], np.array(c["lse"]), 1e-14, c["name"] + " lse")


# ---------------------------------------------------------------------------
# backward pins
# ---------------------------------------------------------------------------

def pin_bwd_finite_differences(orc):
    """Central finite differences of sum(dout * fwd) in float64 match the backward (causal GQA, window, Tq<Tk)."""
    r = _rng(11)
    for (Tq, Tk, window) in [(7, 7, 0), (5, 8, 0), (8, 8, 3)]:
        B, Hq, Hkv, d = 1, 2, 1, 3
        q = r.standard_normal((B, Tq, Hq, d))
        k = r.standard_normal((B, Tk, Hkv, d))
        v = r.standard_normal((B, Tk, Hkv, d))
        P = r.standard_normal((Hq, d, d)) * 0.5
        g = r.standard_normal((B, Tq, Hq, d))
        grads = orc.bwd(q, k, v, P, g, causal=True, window=window)
        eps = 1e-6
        for idx, x in enumerate((q, k, v, P)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                mi = it.multi_index
                old = x[mi]
                x[mi] = old + eps
                fp = np.sum(g * orc.fwd(q, k, v, P, causal=True, window=window)[0])
                x[mi] = old - eps
                fm = np.sum(g * orc.fwd(q, k, v, P, causal=True, window=window)[0])
                x[mi] = old
                num[mi] = (fp - fm) / (2 * eps)
            _close(grads[idx], num, 2e-7, f"finite differences arg {idx} Tq={Tq} Tk={Tk} W={window}")


def _torch_forward(q, k, v, P, causal, scale):
    """Independent autograd-friendly torch forward (dense masked softmax, covariance applied to the probe)."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    K = k.repeat_interleave(Hq // Hkv, dim=2)
    V = v.repeat_interleave(Hq // Hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", q, K) * scale
    if causal:
        i = torch.arange(Tq)[:, None] + (Tk - Tq)
        j = torch.arange(Tk)[None, :]
        s = s.masked_fill(j > i, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, V)
    kb = torch.einsum("bhij,bjhd->bihd", p, K)
    u = torch.einsum("bihc,hca->biha", q - kb, P)
    Kc = K[:, None, :, :, :] - kb[:, :, None, :, :]          # b i j h d
    Vc = V[:, None, :, :, :] - o[:, :, None, :, :]
    t = torch.einsum("biha,bijha->bhij", u, Kc)
    return o + torch.einsum("bhij,bijhd->bihd", p * t, Vc)


def pin_bwd_autograd(orc):
    """torch.autograd (float64) through an independent dense torch forward matches the backward."""
    q, k, v, P = _rand_case(12, B=2, Tq=10, Tk=13, Hq=4, Hkv=2, d=5, p_std=0.4)
    g = _rng(13).standard_normal(q.shape)
    T = [torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v, P)]
    out = _torch_forward(*T, causal=True, scale=1.0 / math.sqrt(5))
    out.backward(torch.from_numpy(g))
    grads = orc.bwd(q, k, v, P, g, causal=True)
    for name, a, t in zip("qkvP", grads, T):
        _close(a, t.grad.numpy(), 1e-11, f"autograd d{name}")


def pin_bwd_zero_projector_is_sdpa(orc):
    """P = 0: dq, dk, dv equal torch SDPA's backward; dP equals sum_i (q_i - kbar_i) du_i^T."""
    q, k, v, P = _rand_case(14, B=1, Tq=12, Tk=12, Hq=4, Hkv=2, d=6)
    g = _rng(15).standard_normal(q.shape)
    d = q.shape[-1]
    Q = torch.from_numpy(q.copy()).permute(0, 2, 1, 3).requires_grad_(True)
    Kt = torch.from_numpy(k.copy()).requires_grad_(True)
    Vt = torch.from_numpy(v.copy()).requires_grad_(True)
    K = Kt.permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    V = Vt.permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
    o.permute(0, 2, 1, 3).backward(torch.from_numpy(g))
    dq, dk, dv, dP = orc.bwd(q, k, v, np.zeros_like(P), g, causal=True)
    _close(dq, Q.grad.permute(0, 2, 1, 3).numpy(), 1e-12, "P=0 dq")
    _close(dk, Kt.grad.numpy(), 1e-12, "P=0 dk")
    _close(dv, Vt.grad.numpy(), 1e-12, "P=0 dv")
    # dP at P = 0 from first principles: u is linear in P, so d out / dP only acts through c = Sigma_KV u.
    scale = 1.0 / math.sqrt(d)
    want = np.zeros_like(P)
    for h in range(4):
        for i in range(12):
            Kj, Vj = k[0, :i + 1, h // 2], v[0, :i + 1, h // 2]
            p = scipy.special.softmax(scale * (Kj @ q[0, i, h]))
            kb = np.average(Kj, axis=0, weights=p)
            cov = _weighted_cov(Vj, Kj, p)                       # d out / d u = cov
            du = cov.T @ g[0, i, h]
            want[h] += np.outer(q[0, i, h] - kb, du)
    _close(dP, want, 1e-11, "P=0 dP")


# ---------------------------------------------------------------------------
# decode pins
# ---------------------------------------------------------------------------

def pin_decode(orc):
    """Decode: P = 0 equals SDPA of the query against its cache prefix; with P it equals the last forward row."""
    r = _rng(16)
    B, L, Hq, Hkv, d = 3, 14, 4, 2, 5
    q = r.standard_normal((B, Hq, d))
    kc = r.standard_normal((B, L, Hkv, d))
    vc = r.standard_normal((B, L, Hkv, d))
    P = r.standard_normal((Hq, d, d)) * 0.4
    seqlens = np.array([14, 1, 9])
    out0 = orc.decode(q, kc, vc, np.zeros_like(P), seqlens=seqlens)
    for b in range(B):
        Lb = seqlens[b]
        ref = _sdpa(q[b:b + 1, None], kc[b:b + 1, :Lb], vc[b:b + 1, :Lb], False, 1.0 / math.sqrt(d))
        _close(out0[b], ref[0, 0], 1e-12, f"decode P=0 batch {b}")
    out = orc.decode(q, kc, vc, P, seqlens=seqlens)
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        Lb = seqlens[b]
        for h in range(Hq):
            Kj, Vj = kc[b, :Lb, h // 2], vc[b, :Lb, h // 2]
            p = scipy.special.softmax(scale * (Kj @ q[b, h]))
            o = np.average(Vj, axis=0, weights=p)
            kb = np.average(Kj, axis=0, weights=p)
            want = o + _weighted_cov(Vj, Kj, p) @ (P[h].T @ (q[b, h] - kb))
            _close(out[b, h], want, 1e-10, f"decode batch {b} head {h}")


def pin_decode_paged(orc):
    """A shuffled page pool with its block table gives exactly ``decode`` on the contiguous cache:
    pages of 4 keys, ragged lengths ending inside a page (and 0), with and without a window."""
    r = _rng(17)
    B, L, Hq, Hkv, d, page = 3, 14, 4, 2, 5, 4
    q = r.standard_normal((B, Hq, d))
    kc = r.standard_normal((B, L, Hkv, d))
    vc = r.standard_normal((B, L, Hkv, d))
    P = r.standard_normal((Hq, d, d)) * 0.4
    seqlens = np.array([14, 7, 0])
    npb = (L + page - 1) // page                                 # pages per sequence
    perm = r.permutation(B * npb + 3)                            # pool with 3 spare pages
    pool_k = r.standard_normal((B * npb + 3, page, Hkv, d))     # spare slots hold junk
    pool_v = r.standard_normal((B * npb + 3, page, Hkv, d))
    table = np.zeros((B, npb), dtype=np.int64)
    for b in range(B):
        for t in range(npb):
            pg = perm[b * npb + t]
            table[b, t] = pg
            n = min(page, L - t * page)
            pool_k[pg, :n] = kc[b, t * page:t * page + n]
            pool_v[pg, :n] = vc[b, t * page:t * page + n]
    got = orc.decode_paged(q, pool_k, pool_v, table, P, seqlens=seqlens, seqlen_k=L)
    want = orc.decode(q, kc, vc, P, seqlens=seqlens)
    _close(got, want, 0.0, "paged decode vs contiguous")
    W = 5
    got = orc.decode_paged(q, pool_k, pool_v, table, P, seqlens=seqlens, seqlen_k=L, window=W)
    for b in range(B):
        Lb = seqlens[b]
        if Lb == 0:
            _close(got[b], 0.0, 0.0, "paged decode empty sequence")
            continue
        lo = max(0, Lb - W)
        want = orc.decode(q[b:b + 1], kc[b:b + 1, lo:Lb], vc[b:b + 1, lo:Lb], P)
        _close(got[b], want[0], 0.0, f"paged decode window batch {b}")


# ---------------------------------------------------------------------------
# probe-form pins (out_i = o_i - Sigma_KV^(i) rho_i with rho supplied per row)
# ---------------------------------------------------------------------------

def pin_probe_zero_is_sdpa(orc):
    """rho = 0 leaves softmax attention (torch SDPA in float64), causal and not, GQA."""
    q, k, v, _ = _rand_case(21)
    scale = 1.0 / math.sqrt(q.shape[-1])
    for causal in (True, False):
        out = orc.fwd_probe(q, k, v, np.zeros_like(q), causal=causal)[0]
        _close(out, _sdpa(q, k, v, causal, scale), 1e-12, f"probe rho=0 causal={causal}")


def pin_probe_covariance_matrix(orc):
    """out_i = o_i - Sigma_KV^(i) rho_i with Sigma_KV^(i) built by numpy.cov (aweights = p) and a random
    rho, with a window, GQA 4 query heads on 2 key/value heads."""
    q, k, v, _ = _rand_case(22, B=1, Tq=9, Tk=12, Hq=4, Hkv=2, d=5)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    rho = _rng(23).standard_normal(q.shape)
    window = 5
    out = orc.fwd_probe(q, k, v, rho, causal=True, window=window)[0]
    for h in range(4):
        g = h // 2
        for i in range(q.shape[1]):
            ip = i + 3
            lo = max(0, ip - window + 1)
            Kj, Vj = k[0, lo:ip + 1, g], v[0, lo:ip + 1, g]
            p = scipy.special.softmax(scale * (Kj @ q[0, i, h]))
            o = np.average(Vj, axis=0, weights=p)
            want = o - _weighted_cov(Vj, Kj, p) @ rho[0, i, h]
            _close(out[0, i, h], want, 1e-10, f"probe covariance head {h} row {i}")


def pin_probe_matches_projector_form(orc):
    """With rho_i = -P_h^T (q_i - kbar_i), kbar taken from the projector form, the probe form reproduces it."""
    q, k, v, P = _rand_case(24, p_std=0.7)
    out, lse, kbar, o = orc.fwd(q, k, v, P, causal=True, window=7)
    rho = -np.einsum("bthx,hxa->btha", q - kbar, P)
    out2, lse2, o2, rk = orc.fwd_probe(q, k, v, rho, causal=True, window=7)
    _close(out2, out, 1e-12, "probe form vs projector form")
    _close(lse2, lse, 1e-12, "probe form lse")
    _close(o2, o, 1e-12, "probe form softmax output")
    _close(rk, np.einsum("bthd,bthd->bht", rho, kbar), 1e-12, "probe form rho . kbar")


def pin_probe_constant_values(orc):
    """Constant values: the covariance is zero, so the output is that value for any probe."""
    q, k, v, _ = _rand_case(25)
    v[:] = v[:, :1]
    rho = 5.0 * _rng(26).standard_normal(q.shape)
    out = orc.fwd_probe(q, k, v, rho, causal=True)[0]
    for h in range(q.shape[2]):
        _close(out[:, :, h], np.broadcast_to(v[:, :1, h // 2], out[:, :, h].shape), 1e-12, "probe constant V")


def pin_probe_bwd_finite_differences(orc):
    """Central finite differences of sum(dout * fwd_probe) in float64 match bwd_probe for q, k, v and rho
    (causal GQA, a window, more keys than queries)."""
    r = _rng(27)
    for (Tq, Tk, window) in [(7, 7, 0), (5, 8, 0), (8, 8, 3)]:
        B, Hq, Hkv, d = 1, 2, 1, 3
        q = r.standard_normal((B, Tq, Hq, d))
        k = r.standard_normal((B, Tk, Hkv, d))
        v = r.standard_normal((B, Tk, Hkv, d))
        rho = r.standard_normal((B, Tq, Hq, d))
        g = r.standard_normal((B, Tq, Hq, d))
        grads = orc.bwd_probe(q, k, v, rho, g, causal=True, window=window)
        eps = 1e-6
        for idx, x in enumerate((q, k, v, rho)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                mi = it.multi_index
                old = x[mi]
                x[mi] = old + eps
                fp = np.sum(g * orc.fwd_probe(q, k, v, rho, causal=True, window=window)[0])
                x[mi] = old - eps
                fm = np.sum(g * orc.fwd_probe(q, k, v, rho, causal=True, window=window)[0])
                x[mi] = old
                num[mi] = (fp - fm) / (2 * eps)
            _close(grads[idx], num, 2e-7, f"probe finite differences arg {idx} Tq={Tq} Tk={Tk} W={window}")


def _torch_probe_forward(q, k, v, rho, causal, scale):
    """Independent dense torch forward of the probe form: o minus the covariance matrix applied to rho."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    K = k.repeat_interleave(Hq // Hkv, dim=2)
    V = v.repeat_interleave(Hq // Hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", q, K) * scale
    if causal:
        i = torch.arange(Tq)[:, None] + (Tk - Tq)
        j = torch.arange(Tk)[None, :]
        s = s.masked_fill(j > i, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, V)
    kb = torch.einsum("bhij,bjhd->bihd", p, K)
    Kc = K[:, None, :, :, :] - kb[:, :, None, :, :]          # b i j h d
    Vc = V[:, None, :, :, :] - o[:, :, None, :, :]
    sigma = torch.einsum("bhij,bijhx,bijhy->bihxy", p, Vc, Kc)   # Sigma_KV per row: [b i h d_v d_k]
    return o - torch.einsum("bihxy,bihy->bihx", sigma, rho)


def pin_probe_bwd_autograd(orc):
    """torch.autograd (float64) through an independent dense torch forward of the probe form matches bwd_probe."""
    q, k, v, _ = _rand_case(28, B=2, Tq=10, Tk=13, Hq=4, Hkv=2, d=5)
    rho = 0.7 * _rng(29).standard_normal(q.shape)
    g = _rng(30).standard_normal(q.shape)
    T = [torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v, rho)]
    out = _torch_probe_forward(*T, causal=True, scale=1.0 / math.sqrt(5))
    out.backward(torch.from_numpy(g))
    grads = orc.bwd_probe(q, k, v, rho, g, causal=True)
    for name, a, t in zip(("q", "k", "v", "rho"), grads, T):
        _close(a, t.grad.numpy(), 1e-11, f"probe autograd d{name}")


def pin_probe_bwd_sdpa_and_covariance(orc):
    """rho = 0: dq, dk, dv equal torch SDPA's backward.  For any rho, out is linear in rho with slope
    -Sigma_KV^(i), so drho_i = -Sigma_KV^(i)T dout_i (Sigma_KV built with numpy.cov, aweights = p)."""
    q, k, v, _ = _rand_case(31, B=1, Tq=12, Tk=12, Hq=4, Hkv=2, d=6)
    g = _rng(32).standard_normal(q.shape)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    Q = torch.from_numpy(q.copy()).permute(0, 2, 1, 3).requires_grad_(True)
    Kt = torch.from_numpy(k.copy()).requires_grad_(True)
    Vt = torch.from_numpy(v.copy()).requires_grad_(True)
    K = Kt.permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    V = Vt.permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
    o.permute(0, 2, 1, 3).backward(torch.from_numpy(g))
    dq, dk, dv, _ = orc.bwd_probe(q, k, v, np.zeros_like(q), g, causal=True)
    _close(dq, Q.grad.permute(0, 2, 1, 3).numpy(), 1e-12, "rho=0 dq")
    _close(dk, Kt.grad.numpy(), 1e-12, "rho=0 dk")
    _close(dv, Vt.grad.numpy(), 1e-12, "rho=0 dv")
    rho = _rng(33).standard_normal(q.shape)
    drho = orc.bwd_probe(q, k, v, rho, g, causal=True)[3]
    for h in range(4):
        for i in range(12):
            Kj, Vj = k[0, :i + 1, h // 2], v[0, :i + 1, h // 2]
            p = scipy.special.softmax(scale * (Kj @ q[0, i, h]))
            want = -_weighted_cov(Vj, Kj, p).T @ g[0, i, h]
            _close(drho[0, i, h], want, 1e-12, f"drho head {h} row {i}")


PROBE_PINS = [pin_probe_zero_is_sdpa, pin_probe_covariance_matrix, pin_probe_matches_projector_form,
              pin_probe_constant_values, pin_probe_bwd_finite_differences, pin_probe_bwd_autograd,
              pin_probe_bwd_sdpa_and_covariance]


FORWARD_PINS = [pin_zero_projector_is_sdpa, pin_bottom_right_alignment, pin_mask_counts,
                pin_exact_lla_is_ridge_wls, pin_covariance_form, pin_constant_values,
                pin_single_key_rows, pin_affine_values, pin_linear_in_projector, pin_hand_examples]
BACKWARD_PINS = [pin_bwd_finite_differences, pin_bwd_autograd, pin_bwd_zero_projector_is_sdpa]
DECODE_PINS = [pin_decode, pin_decode_paged]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS + DECODE_PINS + PROBE_PINS
