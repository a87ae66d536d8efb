"""The no-allocation decode entry point against the workspace one, through the C ABI (GPU)."""
import pytest
import torch

import workloads as W
from tests.util import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plx():
    ensure_built()
    import softmax_learned_covariance_amd as m
    return m


def _pair(plx, q, kc, vc, P, **kw):
    ref = plx.parallax_attn_decode(q, kc, vc, P, **kw)
    got = plx.parallax_attn_decode_noalloc(q, kc, vc, P, **kw)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_decode(plx):
    """Two calls in a row, the second smaller (the scratch keeps the first call's contents), then several new
    tokens per sequence with ragged lengths and a window: bit-identical to parallax_attn_decode (same
    kernels, same scratch layout)."""
    print("[no-alloc] B=64 L=4096 then B=5 L=1500", flush=True)
    w1 = W.scaled(W.WORKLOADS["decode"], batch=64, seqlen_k=4096)
    q, kc, vc, P = W.make_inputs(w1, device="cuda")
    ref, got = _pair(plx, q, kc, vc, P)
    assert torch.equal(ref, got)
    w2 = W.scaled(W.WORKLOADS["decode"], batch=5, seqlen_k=1500)
    q2, kc2, vc2, P2 = W.make_inputs(w2, device="cuda")
    seqlens = torch.tensor([1500, 1, 0, 777, 1024], dtype=torch.int32, device="cuda")
    ref, got = _pair(plx, q2, kc2, vc2, P2, seqlens=seqlens, window=100)
    assert torch.equal(ref, got)
    print("[no-alloc] three new tokens per sequence, preallocated out", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    q3 = torch.randn((5, 3, w2.heads_q, w2.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    ref = plx.parallax_attn_decode(q3, kc2, vc2, P2, seqlens=seqlens)
    out = torch.empty_like(ref)
    got = plx.parallax_attn_decode_noalloc(q3, kc2, vc2, P2, seqlens=seqlens, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(ref, got)


def test_noalloc_rejects_oversized(plx):
    """A decode whose scratch would exceed the fixed array is refused before anything is launched."""
    print("[no-alloc] oversized request", flush=True)
    lib = plx.get_lib()
    cap = lib.parallax_attn_decode_noalloc_max_scratch()
    desc = plx.make_desc(4096, 8, 32768, 16, 8, 128, True, 0, None, plx.PLX_BF16)
    assert lib.parallax_attn_decode_workspace(desc) > cap
    fake = torch.empty(16, device="cuda")   # never dereferenced: the size check comes first
    import ctypes
    st = lib.parallax_attn_decode_noalloc(ctypes.byref(desc), ctypes.c_void_p(fake.data_ptr()),
                                          ctypes.c_void_p(fake.data_ptr()), ctypes.c_void_p(fake.data_ptr()), None,
                                          ctypes.c_void_p(fake.data_ptr()), ctypes.c_void_p(fake.data_ptr()), None,
                                          None)
    assert st == plx.PLX_ERR_WORKSPACE
    assert b"scratch" in lib.parallax_last_error()
