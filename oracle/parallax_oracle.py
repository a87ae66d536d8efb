"""CPU oracle for the Parallax attention operator (test infrastructure only).

Plain, slow, float64 numpy (a float32 mode exists for the CPU timing baseline
only; every parity check runs in float64).  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module; the GPU library never
does, and this module imports nothing from it.

What is computed, per batch b, query head h (key/value head g = h // (Hq/Hkv))
and query row i with visible key set J_i:

  s_ij  = scale * q_i . k_j                       (scale = 1/sqrt(d) by default)
  p_ij  = softmax over j in J_i of s_ij
  o_i   = sum_j p_ij v_j                          softmax attention output
  kbar_i= sum_j p_ij k_j                          softmax-weighted key mean
  u_i   = P_h^T (q_i - kbar_i)                    u_i[a] = sum_b P_h[b][a] (q_i - kbar_i)[b]
  out_i = o_i + sum_j p_ij (u_i . (k_j - kbar_i)) (v_j - o_i)

Sources: the gist.science technical summary of "Parallax: Parameterized Local
Linear Attention for Language Modeling", section "Core mechanism": the output
is the softmax-attention output plus the key/value covariance of the query's
softmax neighbourhood applied to a probe vector (printed as o^SA - Sigma_KV rho;
with rho = -u this is the + form above), and the probe replaces the per-query
solve that exact local linear attention needs (the solve inverts the key
covariance).  The probe's form u = P^T (q - kbar) with one learned d x d
projector P per query head is the reading this operator takes (the pages only
say that a learned map produces the probe); the same section says the boundary
amplification factor eta is set to zero, so no eta term appears.  Setting P = 0
gives plain softmax attention (encorp.ai blog, "Parallax keeps softmax", and the
FAQ answer on converting a pretrained Transformer).

Masks are bottom-right aligned: with offset = Tk - Tq, key j is visible to
query i iff (not causal or j <= i + offset) and (window <= 0 or
j > i + offset - window).  A decode query is the newest token: it sees every
key of its sequence.

Each function also states which tests pin it.  Parity: every function here is
pinned (see the module docstrings of tests/test_oracle_pins.py).
"""
from __future__ import annotations

import contextlib

import numpy as np

ROW_BLOCK = 256


_WORK_DTYPE = np.float64


def _as_f64(x):
    """The working precision of every function here: float64 unless `precision` says otherwise."""
    return np.asarray(x, dtype=_WORK_DTYPE)


@contextlib.contextmanager
def precision(dtype):
    """Runs the oracle's arithmetic in `dtype` inside the block (np.float32 for the CPU timing baseline;
    the default float64 is what every test uses)."""
    global _WORK_DTYPE
    old = _WORK_DTYPE
    _WORK_DTYPE = np.dtype(dtype).type
    try:
        yield
    finally:
        _WORK_DTYPE = old


def visible_range(i: int, Tq: int, Tk: int, causal: bool, window: int):
    """Half-open range [lo, hi) of keys that query row i sees (bottom-right aligned mask)."""
    off = Tk - Tq
    hi = min(Tk, i + off + 1) if causal else Tk
    lo = max(0, i + off - window + 1) if window > 0 else 0
    return lo, max(lo, hi)


def _softmax_rows(s, mask):
    """Softmax of each row over its visible entries; rows with no visible key give all-zero weights."""
    if s.shape[1] == 0:   # a block of rows none of which sees a key
        return np.zeros_like(s), np.full(s.shape[0], -np.inf, dtype=s.dtype)
    s = np.where(mask, s, -np.inf)
    mx = np.max(s, axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.where(mask, np.exp(s - mx), 0.0)
    den = e.sum(axis=1, keepdims=True)
    p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
    lse = np.where(den[:, 0] > 0, mx[:, 0] + np.log(np.where(den[:, 0] > 0, den[:, 0], 1.0)), -np.inf)
    return p, lse


def _row_blocks(Tq, Tk, causal, window, rows):
    """Yield (query-row index array, lo, hi) groups covering the requested rows."""
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    for b0 in range(0, len(rows), ROW_BLOCK):
        rr = rows[b0:b0 + ROW_BLOCK]
        ranges = [visible_range(int(i), Tq, Tk, causal, window) for i in rr]
        lo = min(r[0] for r in ranges)
        hi = max(r[1] for r in ranges)
        yield rr, lo, max(lo, hi)


def _mask_rows(rr, lo, hi, Tq, Tk, causal, window):
    off = Tk - Tq
    i = rr[:, None] + off
    j = np.arange(lo, hi)[None, :]
    m = np.ones((len(rr), hi - lo), dtype=bool)
    if causal:
        m &= j <= i
    if window > 0:
        m &= j > i - window
    return m


def fwd(q, k, v, P, causal=True, window=0, scale=None, rows=None):
    """Parallax forward.

    q [B,Tq,Hq,d]; k, v [B,Tk,Hkv,d]; P [Hq,d,d] (one projector per query head)
    or [B,Tq,Hq,d,d] (one per query, used only for the exact-LLA check case).
    ``rows`` restricts the computation to a subset of query rows (the others
    are returned as NaN), which lets tests sample rows of full-size problems.

    Returns float64 arrays out [B,Tq,Hq,d], lse [B,Hq,Tq] (natural log of the
    softmax denominator, scores scaled), kbar [B,Tq,Hq,d], o [B,Tq,Hq,d].
    Pinned by: P=0 vs torch SDPA; exact-LLA vs brute-force ridge WLS; constant
    and affine V; first causal row and window=1; weighted-covariance form
    (numpy.cov) with rank-one projectors; linearity in P; mask counts.
    """
    q, k, v, P = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(P)
    B, Tq, Hq, d = q.shape
    _, Tk, Hkv, _ = k.shape
    assert Hq % Hkv == 0
    grp = Hq // Hkv
    per_query = P.ndim == 5
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    out = np.full(q.shape, np.nan, dtype=q.dtype)
    kbar = np.full(q.shape, np.nan, dtype=q.dtype)
    osa = np.full(q.shape, np.nan, dtype=q.dtype)
    lse = np.full((B, Hq, Tq), np.nan, dtype=q.dtype)
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            K, V = k[b, :, g, :], v[b, :, g, :]
            for rr, lo, hi in _row_blocks(Tq, Tk, causal, window, rows):
                Qr = q[b, rr, h, :]
                mask = _mask_rows(rr, lo, hi, Tq, Tk, causal, window)
                Kj, Vj = K[lo:hi], V[lo:hi]
                p, l = _softmax_rows(scale * (Qr @ Kj.T), mask)
                o = p @ Vj
                kb = p @ Kj
                x = Qr - kb
                if per_query:
                    u = np.einsum("ib,iba->ia", x, P[b, rr, h])
                else:
                    u = x @ P[h]                                   # u[a] = sum_b x[b] P[b][a]
                # t_ij = u_i . (k_j - kbar_i); centred value v_j - o_i
                t = u @ Kj.T - np.sum(u * kb, axis=1, keepdims=True)
                w = p * t
                c = w @ Vj - np.sum(w, axis=1, keepdims=True) * o   # sum_j w_ij (v_j - o_i)
                out[b, rr, h] = o + c
                kbar[b, rr, h] = kb
                osa[b, rr, h] = o
                lse[b, h, rr] = l
    return out, lse, kbar, osa


def fwd_probe(q, k, v, rho, causal=True, window=0, scale=None, rows=None):
    """Parallax forward with the probe supplied per query row, the pages' own form.

    gist.science technical summary, "Core mechanism": out_i = o^SA_i - Sigma_KV^(i) rho_i, where the
    probe rho_i = W_R x_i is a learned map of the layer input (computed here by the caller) and
    Sigma_KV^(i) is the key/value covariance of the query's softmax neighbourhood, read as
    Sigma_KV^(i) = sum_j p_ij (v_j - o_i)(k_j - kbar_i)^T.  So
      out_i = o_i - sum_j p_ij (rho_i . (k_j - kbar_i)) (v_j - o_i),
    which is fwd() with u_i = -rho_i.

    q, rho [B,Tq,Hq,d]; k, v [B,Tk,Hkv,d].  Returns float64 out [B,Tq,Hq,d], lse [B,Hq,Tq], the
    softmax output o [B,Tq,Hq,d] and rk [B,Hq,Tq] = rho_i . kbar_i (rows outside ``rows`` are NaN);
    o and rk are what ``bwd_probe`` needs besides lse.
    Pinned by: rho = 0 vs torch SDPA; rho = -u of fwd() reproduces fwd(); the covariance matrix
    built with numpy.cov (aweights = p) applied to rho; constant V.
    """
    q, k, v, rho = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(rho)
    B, Tq, Hq, d = q.shape
    _, Tk, Hkv, _ = k.shape
    assert Hq % Hkv == 0 and rho.shape == q.shape
    grp = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    out = np.full(q.shape, np.nan, dtype=q.dtype)
    osa = np.full(q.shape, np.nan, dtype=q.dtype)
    lse = np.full((B, Hq, Tq), np.nan, dtype=q.dtype)
    rk = np.full((B, Hq, Tq), np.nan, dtype=q.dtype)
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            K, V = k[b, :, g, :], v[b, :, g, :]
            for rr, lo, hi in _row_blocks(Tq, Tk, causal, window, rows):
                Qr, Rr = q[b, rr, h, :], rho[b, rr, h, :]
                mask = _mask_rows(rr, lo, hi, Tq, Tk, causal, window)
                Kj, Vj = K[lo:hi], V[lo:hi]
                p, l = _softmax_rows(scale * (Qr @ Kj.T), mask)
                o = p @ Vj
                kb = p @ Kj
                t = Rr @ Kj.T - np.sum(Rr * kb, axis=1, keepdims=True)      # rho_i . (k_j - kbar_i)
                w = p * t
                out[b, rr, h] = o - (w @ Vj - np.sum(w, axis=1, keepdims=True) * o)
                osa[b, rr, h] = o
                lse[b, h, rr] = l
                rk[b, h, rr] = np.sum(Rr * kb, axis=1)
    return out, lse, osa, rk


def bwd_probe(q, k, v, rho, dout, causal=True, window=0, scale=None):
    """Gradients of sum(dout * out) of ``fwd_probe`` with respect to q, k, v and rho.

    The pages give no backward.  Written in the probe's own terms, with r_ij = rho_i . k_j and
    a_i = rho_i . kbar_i = sum_j p_ij r_ij, the forward is
      out_i = (1 + a_i) o_i - sum_j p_ij r_ij v_j
    (the centrings of the covariance cancel against sum_j p_ij (v_j - o_i) = 0).  With g = dout,
    G_ij = g_i . v_j and go_i = g_i . o_i, differentiating through p, o, a and r:
      drho_i = go_i kbar_i - sum_j p_ij G_ij k_j
      dv_j   = sum_i p_ij (1 + a_i - r_ij) g_i
      dp_ij  = G_ij (1 + a_i - r_ij) + go_i r_ij          (a and o depend on p too)
      ds_ij  = p_ij (dp_ij - sum_l p_il dp_il)
      dq_i   = scale sum_j ds_ij k_j
      dk_j   = sum_i [p_ij (go_i - G_ij) rho_i + scale ds_ij q_i]
    dk, dv are summed over the query heads sharing a key/value head.
    Pinned by: central finite differences of ``fwd_probe``; torch.autograd of an independent torch
    forward; rho = 0 against torch SDPA's backward.
    """
    q, k, v, rho, g_all = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(rho), _as_f64(dout)
    B, Tq, Hq, d = q.shape
    _, Tk, Hkv, _ = k.shape
    grp = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    drho = np.zeros_like(rho)
    for b in range(B):
        for h in range(Hq):
            gk = h // grp
            K, V = k[b, :, gk, :], v[b, :, gk, :]
            for rr, lo, hi in _row_blocks(Tq, Tk, causal, window, None):
                Qr, Rr, G = q[b, rr, h, :], rho[b, rr, h, :], g_all[b, rr, h, :]
                mask = _mask_rows(rr, lo, hi, Tq, Tk, causal, window)
                Kj, Vj = K[lo:hi], V[lo:hi]
                p, _ = _softmax_rows(scale * (Qr @ Kj.T), mask)
                o = p @ Vj
                kb = p @ Kj
                r = Rr @ Kj.T                                    # r_ij = rho_i . k_j
                a = np.sum(p * r, axis=1, keepdims=True)         # a_i = rho_i . kbar_i
                gv = G @ Vj.T                                    # G_ij = g_i . v_j
                go = np.sum(G * o, axis=1, keepdims=True)        # go_i = g_i . o_i
                drho[b, rr, h] = go * kb - (p * gv) @ Kj
                dv[b, lo:hi, gk] += (p * (1.0 + a - r)).T @ G
                dp = gv * (1.0 + a - r) + go * r
                ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
                dq[b, rr, h] = scale * (ds @ Kj)
                dk[b, lo:hi, gk] += (p * (go - gv)).T @ Rr + scale * (ds.T @ Qr)
    return dq, dk, dv, drho


def bwd(q, k, v, P, dout, causal=True, window=0, scale=None):
    """Gradients of sum(dout * out) with respect to q, k, v and P (chain rule of ``fwd``).

    The pages give no backward; this is the chain rule of the forward definition,
    written with g = dout, alpha_i = u_i . kbar_i, t_ij = u_i . k_j:
      out_i = (1 - alpha_i) o_i + sum_j p_ij t_ij v_j
      du_i  = sum_j p_ij (g_i.v_j) k_j - (g_i.o_i) kbar_i
      dkbar_i = -(g_i.o_i) u_i - P du_i        dq_i += P du_i     dP += sum_i (q_i - kbar_i) du_i^T
      dp_ij = (g_i.v_j)(t_ij + 1 - alpha_i) + dkbar_i . k_j
      ds_ij = p_ij (dp_ij - sum_l p_il dp_il)
      dq_i += scale sum_j ds_ij k_j
      dk_j += sum_i [p_ij (g_i.v_j) u_i + p_ij dkbar_i + scale ds_ij q_i]
      dv_j += sum_i p_ij (t_ij + 1 - alpha_i) g_i
    dk, dv are summed over the query heads sharing a key/value head; dP over
    batch and rows, in the orientation of P.  Pinned by: central finite
    differences of ``fwd``; torch.autograd of an independent torch forward;
    P=0 against torch SDPA's backward.
    """
    q, k, v, P, g_all = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(P), _as_f64(dout)
    B, Tq, Hq, d = q.shape
    _, Tk, Hkv, _ = k.shape
    grp = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dP = np.zeros_like(P)
    for b in range(B):
        for h in range(Hq):
            gk = h // grp
            K, V = k[b, :, gk, :], v[b, :, gk, :]
            Ph = P[h]
            for rr, lo, hi in _row_blocks(Tq, Tk, causal, window, None):
                Qr, G = q[b, rr, h, :], g_all[b, rr, h, :]
                mask = _mask_rows(rr, lo, hi, Tq, Tk, causal, window)
                Kj, Vj = K[lo:hi], V[lo:hi]
                p, _ = _softmax_rows(scale * (Qr @ Kj.T), mask)
                o = p @ Vj
                kb = p @ Kj
                x = Qr - kb
                u = x @ Ph
                alpha = np.sum(u * kb, axis=1, keepdims=True)
                t = u @ Kj.T
                gv = G @ Vj.T                                    # g_i . v_j
                go = np.sum(G * o, axis=1, keepdims=True)        # g_i . o_i
                du = (p * gv) @ Kj - go * kb
                Pdu = du @ Ph.T                                  # (P du)[b] = sum_a P[b][a] du[a]
                dkb = -go * u - Pdu
                dP[h] += x.T @ du
                dp = gv * (t + 1.0 - alpha) + dkb @ Kj.T
                delta = np.sum(p * dp, axis=1, keepdims=True)
                ds = p * (dp - delta)
                dq[b, rr, h] += Pdu + scale * (ds @ Kj)
                dk[b, lo:hi, gk] += (p * gv).T @ u + p.T @ dkb + scale * (ds.T @ Qr)
                dv[b, lo:hi, gk] += (p * (t + 1.0 - alpha)).T @ G
    return dq, dk, dv, dP


def decode(q, k_cache, v_cache, P, seqlens=None, scale=None):
    """One new query per sequence against a key/value cache.

    q [B,Hq,d]; caches [B,Lmax,Hkv,d]; seqlens [B] (None: every sequence has
    length Lmax).  The new token's key and value are already the last cache
    entry, so query b sees keys 0..seqlens[b]-1.  Equals the last row of
    ``fwd`` over the cache prefix (that is how it is computed here).
    Pinned by: P=0 vs torch SDPA, and (through ``fwd``) all forward pins.
    """
    q = _as_f64(q)
    B, Hq, d = q.shape
    Lmax = k_cache.shape[1]
    out = np.zeros((B, Hq, d), dtype=q.dtype)
    for b in range(B):
        L = Lmax if seqlens is None else int(seqlens[b])
        if L == 0:
            continue
        o, _, _, _ = fwd(q[b:b + 1, None], k_cache[b:b + 1, :L], v_cache[b:b + 1, :L], P,
                         causal=True, window=0, scale=scale)
        out[b] = o[0, 0]
    return out


def decode_paged(q, k_pages, v_pages, block_table, P, seqlens=None, seqlen_k=None, window=0, scale=None):
    """Decode against a paged cache: key j of sequence b is row j % page_size of page
    block_table[b][j // page_size].  Each sequence's keys are gathered through its table into a
    contiguous array (a change of storage only), then the newest ``window`` of them (all when
    window <= 0) go through ``decode``.

    q [B,Hq,d]; pages [num_pages, page_size, Hkv, d]; block_table [B, max_pages] ints; seqlens [B]
    (None: every sequence has seqlen_k = max_pages * page_size keys).  Returns out [B,Hq,d].
    Pinned by: a shuffled page pool with its table equals ``decode`` on the contiguous cache,
    with ragged lengths that end inside a page and a window.
    """
    q = _as_f64(q)
    k_pages, v_pages = _as_f64(k_pages), _as_f64(v_pages)
    block_table = np.asarray(block_table)
    B = q.shape[0]
    page = k_pages.shape[1]
    Lmax = block_table.shape[1] * page if seqlen_k is None else int(seqlen_k)
    out = np.zeros(q.shape, dtype=q.dtype)
    for b in range(B):
        L = Lmax if seqlens is None else min(max(int(seqlens[b]), 0), Lmax)
        lo = max(0, L - window) if window > 0 else 0
        if L - lo == 0:
            continue
        j = np.arange(lo, L)
        pages_of_j = block_table[b, j // page]
        Kb = k_pages[pages_of_j, j % page]                     # [L - lo, Hkv, d]
        Vb = v_pages[pages_of_j, j % page]
        out[b] = decode(q[b:b + 1], Kb[None], Vb[None], P, scale=scale)[0]
    return out


def exact_lla_projector(q, k, causal=True, window=0, scale=None, lam=1e-2):
    """Per-query projector P_i = (Sigma_q,i + lam I)^-1 that turns the operator into exact ridge LLA.

    Sigma_q,i = sum_j p_ij (k_j - kbar_i)(k_j - kbar_i)^T is the softmax-weighted
    key covariance of query i (the matrix exact local linear attention inverts,
    per the "Core mechanism" section cited in the module docstring).  With this
    P (symmetric, so P^T = P) the output is the intercept of the weighted ridge
    regression of the values on the keys centred at the query.
    Returns [B,Tq,Hq,d,d] float64.
    """
    q, k = _as_f64(q), _as_f64(k)
    B, Tq, Hq, d = q.shape
    _, Tk, Hkv, _ = k.shape
    grp = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    Pq = np.zeros((B, Tq, Hq, d, d))
    for b in range(B):
        for h in range(Hq):
            K = k[b, :, h // grp, :]
            for i in range(Tq):
                lo, hi = visible_range(i, Tq, Tk, causal, window)
                Kj = K[lo:hi]
                s = scale * (Kj @ q[b, i, h])
                p = np.exp(s - s.max())
                p /= p.sum()
                kb = p @ Kj
                Kc = Kj - kb
                cov = (Kc * p[:, None]).T @ Kc
                Pq[b, i, h] = np.linalg.inv(cov + lam * np.eye(d))
    return Pq
