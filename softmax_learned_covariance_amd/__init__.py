"""Parallax attention on AMD Instinct MI355X: thin Python binding of libparallax.so.

The binding only marshals arguments: it checks shapes and dtypes, allocates the
output tensors and the workspace with PyTorch, and calls the C entry points
declared in include/parallax.h on the current HIP stream.  Every step of the
operator runs in the library's HIP kernels; there is no Python or CPU fallback,
and the first call raises ImportError when the library has not been built
(``python -m softmax_learned_covariance_amd.build``).

Functions (same names as the C entry points):

    out, lse, kbar, o = parallax_attn_fwd(q, k, v, P, causal=True, window=0, scale=None)
    dq, dk, dv, dP    = parallax_attn_bwd(q, k, v, P, out, dout, lse, kbar, o, causal=True, ...)
    out               = parallax_attn_decode(q, k_cache, v_cache, P, seqlens=None, window=0, scale=None)
    out, lse, o, rk   = parallax_attn_fwd_probe(q, k, v, rho, causal=True, window=0, scale=None)
    dq, dk, dv, drho  = parallax_attn_bwd_probe(q, k, v, rho, out, dout, lse, o, rk, causal=True, ...)
    out               = parallax_attn_decode_paged(q, k_pages, v_pages, block_table, P, seqlens=None, ...)
    out               = parallax_attn_decode_noalloc(q, k_cache, v_cache, P, seqlens=None, ...)  (no workspace)
    parallax_set_decode_path(PLX_DECODE_TWO_PASS)   (process-wide decode kernel choice; PLX_DECODE_AUTO default)

Layouts: q [B,Tq,Hq,d] (decode [B,Hq,d]); k, v [B,Tk,Hkv,d]; P [Hq,d,d] (or
[B,Tq,Hq,d,d] per query, forward only); outputs float32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libparallax.so")

PLX_OK, PLX_ERR_INVALID, PLX_ERR_UNSUPPORTED, PLX_ERR_WORKSPACE, PLX_ERR_HIP = range(5)
PLX_F32, PLX_BF16 = 0, 1
(PLX_KERNEL_FWD, PLX_KERNEL_BWD_ROWS, PLX_KERNEL_BWD_KEYS, PLX_KERNEL_DECODE_PASS1, PLX_KERNEL_DECODE_PASS2,
 PLX_KERNEL_BWD_DQ, PLX_KERNEL_FWD_PROBE, PLX_KERNEL_DECODE_MOMENT) = range(8)
PLX_DECODE_AUTO, PLX_DECODE_TWO_PASS = 0, 1


class PlxAttnDesc(ctypes.Structure):
    """Mirror of plx_attn_desc (include/parallax.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
        ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("window", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("p_per_query", ctypes.c_int32), ("split_rows", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
    ]


class ParallaxError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{detail} [status {status}]")
        self.status = status


_vp, _sz, _st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_DESC = ctypes.POINTER(PlxAttnDesc)
SIGNATURES = {
    "parallax_set_kernel_events": (None, [ctypes.c_int, _vp, _vp]),
    "parallax_set_decode_path": (_st, [ctypes.c_int32]),
    "parallax_abi_version": (ctypes.c_int, []),
    "parallax_status_string": (ctypes.c_char_p, [_st]),
    "parallax_last_error": (ctypes.c_char_p, []),
    "parallax_attn_fwd_workspace": (_sz, [_DESC]),
    "parallax_attn_fwd": (_st, [_DESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "parallax_attn_fwd_probe_workspace": (_sz, [_DESC]),
    "parallax_attn_fwd_probe": (_st, [_DESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "parallax_attn_bwd_probe_workspace": (_sz, [_DESC]),
    "parallax_attn_bwd_probe": (_st, [_DESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "parallax_attn_bwd_workspace": (_sz, [_DESC]),
    "parallax_attn_bwd": (_st, [_DESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "parallax_attn_decode_workspace": (_sz, [_DESC]),
    "parallax_attn_decode": (_st, [_DESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "parallax_attn_decode_noalloc_max_scratch": (_sz, []),
    "parallax_attn_decode_noalloc": (_st, [_DESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "parallax_attn_decode_paged_workspace": (_sz, [_DESC]),
    "parallax_attn_decode_paged": (_st, [_DESC, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int32,
                                         _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libparallax.so and declares the C signatures; raises if it is missing."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m softmax_learned_covariance_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def get_lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


def _check(status):
    if status != PLX_OK:
        raise ParallaxError(status, get_lib().parallax_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return PLX_F32
    if t.dtype == torch.bfloat16:
        return PLX_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _need(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def make_desc(B, Tq, Tk, Hq, Hkv, d, causal=True, window=0, scale=None, dtype=PLX_BF16,
              p_per_query=False, split_rows=-1, out_dtype=PLX_F32) -> PlxAttnDesc:
    return PlxAttnDesc(B, Tq, Tk, Hq, Hkv, d, int(bool(causal)), int(window or 0),
                       float(scale) if scale else 0.0, dtype, int(bool(p_per_query)), int(split_rows),
                       int(out_dtype))


def _out_code(out_dtype):
    if out_dtype in (None, torch.float32):
        return PLX_F32, torch.float32
    if out_dtype == torch.bfloat16:
        return PLX_BF16, torch.bfloat16
    raise TypeError(f"out_dtype must be float32 or bfloat16, not {out_dtype}")


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def parallax_attn_fwd(q, k, v, P, causal=True, window=0, scale=None, split_rows=-1, out_dtype=torch.float32,
                      cor=False):
    """Forward; returns (out, lse, kbar, o_sa), float32 (out in `out_dtype`), plus the per-row
    correction-to-output ratio [B,Hq,Tq] when cor=True (see include/parallax.h)."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    per_query = P.dim() == 5
    _need(q, "q", q.dtype, (B, Tq, Hq, d), q.device)
    _need(k, "k", q.dtype, (B, Tk, Hkv, d), q.device)
    _need(v, "v", q.dtype, (B, Tk, Hkv, d), q.device)
    _need(P, "P", q.dtype, (B, Tq, Hq, d, d) if per_query else (Hq, d, d), q.device)
    oc, odt = _out_code(out_dtype)
    desc = make_desc(B, Tq, Tk, Hq, Hkv, d, causal, window, scale, dt, per_query, split_rows, oc)
    f32 = dict(dtype=torch.float32, device=q.device)
    out = torch.empty((B, Tq, Hq, d), dtype=odt, device=q.device)
    lse = torch.empty((B, Hq, Tq), **f32)
    kbar = torch.empty((B, Tq, Hq, d), **f32)
    osa = torch.empty((B, Tq, Hq, d), **f32)
    ratio = torch.empty((B, Hq, Tq), **f32) if cor else None
    lib = get_lib()
    nws = lib.parallax_attn_fwd_workspace(ctypes.byref(desc))
    ws = _workspace(nws, q.device)
    _check(lib.parallax_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(out),
                                 _ptr(lse), _ptr(kbar), _ptr(osa), _ptr(ratio), _ptr(ws), nws, _stream()))
    return (out, lse, kbar, osa, ratio) if cor else (out, lse, kbar, osa)


def parallax_attn_fwd_probe(q, k, v, rho, causal=True, window=0, scale=None, split_rows=-1, out_dtype=torch.float32,
                            cor=False):
    """Probe-form forward, rho [B,Tq,Hq,d] like q; returns (out, lse, o_sa, rk), float32 (out in `out_dtype`),
    plus the correction-to-output ratio when cor=True (see include/parallax.h)."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    _need(k, "k", q.dtype, (B, Tk, Hkv, d), q.device)
    _need(v, "v", q.dtype, (B, Tk, Hkv, d), q.device)
    _need(rho, "rho", q.dtype, (B, Tq, Hq, d), q.device)
    _need(q, "q", q.dtype, (B, Tq, Hq, d), q.device)
    oc, odt = _out_code(out_dtype)
    desc = make_desc(B, Tq, Tk, Hq, Hkv, d, causal, window, scale, dt, False, split_rows, oc)
    f32 = dict(dtype=torch.float32, device=q.device)
    out = torch.empty((B, Tq, Hq, d), dtype=odt, device=q.device)
    lse = torch.empty((B, Hq, Tq), **f32)
    osa = torch.empty((B, Tq, Hq, d), **f32)
    rk = torch.empty((B, Hq, Tq), **f32)
    ratio = torch.empty((B, Hq, Tq), **f32) if cor else None
    lib = get_lib()
    nws = lib.parallax_attn_fwd_probe_workspace(ctypes.byref(desc))
    ws = _workspace(nws, q.device)
    _check(lib.parallax_attn_fwd_probe(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(out),
                                       _ptr(lse), _ptr(osa), _ptr(rk), _ptr(ratio), _ptr(ws), nws, _stream()))
    return (out, lse, osa, rk, ratio) if cor else (out, lse, osa, rk)


def parallax_attn_bwd_probe(q, k, v, rho, out, dout, lse, o_sa, rk, causal=True, window=0, scale=None,
                            split_rows=-1):
    """Probe-form backward; returns (dq, dk, dv, drho), all float32 (see include/parallax.h)."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    dev = q.device
    _need(k, "k", q.dtype, (B, Tk, Hkv, d), dev)
    _need(v, "v", q.dtype, (B, Tk, Hkv, d), dev)
    _need(rho, "rho", q.dtype, (B, Tq, Hq, d), dev)
    _need(dout, "dout", q.dtype, (B, Tq, Hq, d), dev)
    for name, t in (("out", out), ("o_sa", o_sa)):
        _need(t, name, torch.float32, (B, Tq, Hq, d), dev)
    for name, t in (("lse", lse), ("rk", rk)):
        _need(t, name, torch.float32, (B, Hq, Tq), dev)
    desc = make_desc(B, Tq, Tk, Hq, Hkv, d, causal, window, scale, dt, False, split_rows)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, Tq, Hq, d), **f32)
    dk = torch.empty((B, Tk, Hkv, d), **f32)
    dv = torch.empty((B, Tk, Hkv, d), **f32)
    drho = torch.empty((B, Tq, Hq, d), **f32)
    lib = get_lib()
    nws = lib.parallax_attn_bwd_probe_workspace(ctypes.byref(desc))
    ws = _workspace(nws, dev)
    _check(lib.parallax_attn_bwd_probe(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(out),
                                       _ptr(dout), _ptr(lse), _ptr(o_sa), _ptr(rk), _ptr(dq), _ptr(dk),
                                       _ptr(dv), _ptr(drho), _ptr(ws), nws, _stream()))
    return dq, dk, dv, drho


def parallax_attn_bwd(q, k, v, P, out, dout, lse, kbar, o_sa, causal=True, window=0, scale=None,
                      split_rows=-1):
    """Backward; returns (dq, dk, dv, dP), all float32 (see include/parallax.h)."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    dev = q.device
    _need(k, "k", q.dtype, (B, Tk, Hkv, d), dev)
    _need(v, "v", q.dtype, (B, Tk, Hkv, d), dev)
    _need(P, "P", q.dtype, (Hq, d, d), dev)
    _need(dout, "dout", q.dtype, (B, Tq, Hq, d), dev)
    for name, t in (("out", out), ("kbar", kbar), ("o_sa", o_sa)):
        _need(t, name, torch.float32, (B, Tq, Hq, d), dev)
    _need(lse, "lse", torch.float32, (B, Hq, Tq), dev)
    desc = make_desc(B, Tq, Tk, Hq, Hkv, d, causal, window, scale, dt, False, split_rows)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, Tq, Hq, d), **f32)
    dk = torch.empty((B, Tk, Hkv, d), **f32)
    dv = torch.empty((B, Tk, Hkv, d), **f32)
    dP = torch.empty((Hq, d, d), **f32)
    lib = get_lib()
    nws = lib.parallax_attn_bwd_workspace(ctypes.byref(desc))
    ws = _workspace(nws, dev)
    _check(lib.parallax_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(out),
                                 _ptr(dout), _ptr(lse), _ptr(kbar), _ptr(o_sa), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(dP), _ptr(ws), nws, _stream()))
    return dq, dk, dv, dP


def parallax_set_decode_path(path):
    """Selects the decode kernels for the whole process: PLX_DECODE_AUTO (the single-read kernel where it
    applies) or PLX_DECODE_TWO_PASS (always the two split-KV passes)."""
    _check(get_lib().parallax_set_decode_path(int(path)))


def parallax_attn_decode(q, k_cache, v_cache, P, seqlens=None, window=0, scale=None, out_dtype=torch.float32,
                         cor=False):
    """Decode; q [B,Hq,d] (one new token) or [B,T,Hq,d] (the last T tokens of each sequence), caches
    [B,Lmax,Hkv,d], seqlens int32 [B] or None; returns out shaped like q (float32 or `out_dtype`), and the
    correction-to-output ratio (q's shape without d) as well when cor=True."""
    lead = q.shape[:-2]
    B, Hq, d = q.shape[0], q.shape[-2], q.shape[-1]
    T = q.shape[1] if q.dim() == 4 else 1
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    dev = q.device
    _need(k_cache, "k_cache", q.dtype, (B, Lmax, Hkv, d), dev)
    _need(v_cache, "v_cache", q.dtype, (B, Lmax, Hkv, d), dev)
    _need(P, "P", q.dtype, (Hq, d, d), dev)
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, (B,), dev)
    oc, odt = _out_code(out_dtype)
    desc = make_desc(B, T, Lmax, Hq, Hkv, d, True, window, scale, dt, False, -1, oc)
    out = torch.empty((*lead, Hq, d), dtype=odt, device=dev)
    ratio = torch.empty((*lead, Hq), dtype=torch.float32, device=dev) if cor else None
    if not q.is_contiguous():
        raise ValueError("q: must be contiguous")
    lib = get_lib()
    nws = lib.parallax_attn_decode_workspace(ctypes.byref(desc))
    ws = _workspace(nws, dev)
    _check(lib.parallax_attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(seqlens), _ptr(P), _ptr(out), _ptr(ratio), _ptr(ws), nws, _stream()))
    return (out, ratio) if cor else out


def parallax_attn_decode_noalloc(q, k_cache, v_cache, P, seqlens=None, window=0, scale=None, out_dtype=torch.float32,
                                 cor=False, out=None, cor_out=None):
    """Decode through the no-allocation entry point (the library's fixed scratch instead of a workspace):
    arguments and results as parallax_attn_decode.  `out` (and `cor_out` with cor=True) may be given
    preallocated, so that the call allocates nothing at all (e.g. under HIP graph capture)."""
    lead = q.shape[:-2]
    B, Hq, d = q.shape[0], q.shape[-2], q.shape[-1]
    T = q.shape[1] if q.dim() == 4 else 1
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    dev = q.device
    _need(k_cache, "k_cache", q.dtype, (B, Lmax, Hkv, d), dev)
    _need(v_cache, "v_cache", q.dtype, (B, Lmax, Hkv, d), dev)
    _need(P, "P", q.dtype, (Hq, d, d), dev)
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, (B,), dev)
    if not q.is_contiguous():
        raise ValueError("q: must be contiguous")
    oc, odt = _out_code(out_dtype)
    desc = make_desc(B, T, Lmax, Hq, Hkv, d, True, window, scale, dt, False, -1, oc)
    if out is None:
        out = torch.empty((*lead, Hq, d), dtype=odt, device=dev)
    _need(out, "out", odt, (*lead, Hq, d), dev)
    ratio = None
    if cor:
        ratio = cor_out if cor_out is not None else torch.empty((*lead, Hq), dtype=torch.float32, device=dev)
        _need(ratio, "cor_out", torch.float32, (*lead, Hq), dev)
    _check(get_lib().parallax_attn_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                  _ptr(seqlens), _ptr(P), _ptr(out), _ptr(ratio), _stream()))
    return (out, ratio) if cor else out


def parallax_attn_decode_paged(q, k_pages, v_pages, block_table, P, seqlens=None, seqlen_k=None, window=0,
                               scale=None, out_dtype=torch.float32, cor=False):
    """Decode against a paged cache: q [B,Hq,d] or [B,T,Hq,d]; pages [num_pages,page_size,Hkv,d]; block_table
    int32 [B,max_pages] (its width is passed as the row stride, so it may exceed what seqlen_k needs); seqlens int32
    [B] or None; seqlen_k defaults to max_pages * page_size.
    Returns out shaped like q (see include/parallax.h)."""
    lead = q.shape[:-2]
    B, Hq, d = q.shape[0], q.shape[-2], q.shape[-1]
    T = q.shape[1] if q.dim() == 4 else 1
    if not q.is_contiguous():
        raise ValueError("q: must be contiguous")
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    dt = _dtype_code(q)
    dev = q.device
    _need(k_pages, "k_pages", q.dtype, (num_pages, page_size, Hkv, d), dev)
    _need(v_pages, "v_pages", q.dtype, (num_pages, page_size, Hkv, d), dev)
    _need(P, "P", q.dtype, (Hq, d, d), dev)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table: expected int32 [B, max_pages], got {block_table.dtype} {tuple(block_table.shape)}")
    _need(block_table, "block_table", torch.int32, tuple(block_table.shape), dev)
    Lmax = block_table.shape[1] * page_size if seqlen_k is None else int(seqlen_k)
    if (Lmax + page_size - 1) // page_size > block_table.shape[1]:
        raise ValueError(f"seqlen_k={Lmax} needs more than the block table's {block_table.shape[1]} pages")
    if seqlens is not None:
        _need(seqlens, "seqlens", torch.int32, (B,), dev)
    oc, odt = _out_code(out_dtype)
    desc = make_desc(B, T, Lmax, Hq, Hkv, d, True, window, scale, dt, False, -1, oc)
    out = torch.empty((*lead, Hq, d), dtype=odt, device=dev)
    ratio = torch.empty((*lead, Hq), dtype=torch.float32, device=dev) if cor else None
    lib = get_lib()
    nws = lib.parallax_attn_decode_paged_workspace(ctypes.byref(desc))
    ws = _workspace(nws, dev)
    _check(lib.parallax_attn_decode_paged(ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), num_pages,
                                          page_size, _ptr(block_table), block_table.shape[1], _ptr(seqlens),
                                          _ptr(P), _ptr(out),
                                          _ptr(ratio), _ptr(ws), nws, _stream()))
    return (out, ratio) if cor else out


fwd = parallax_attn_fwd
bwd = parallax_attn_bwd
decode = parallax_attn_decode
fwd_probe = parallax_attn_fwd_probe
bwd_probe = parallax_attn_bwd_probe
decode_paged = parallax_attn_decode_paged
decode_noalloc = parallax_attn_decode_noalloc
