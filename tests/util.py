"""Helpers shared by the tests (no operator arithmetic here)."""
import os

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def rel_err(got, ref):
    """max |got - ref| / sqrt(mean(ref^2)) over all elements (the tolerance metric of every parity test)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / rms) if rms > 0 else float(np.max(np.abs(got - ref)))


def sampled_rel_err(got, ref, norm_ref):
    """max |got - ref| over the checked elements, divided by the rms of an unbiased row sample."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    rms = np.sqrt(np.mean(np.asarray(norm_ref, dtype=np.float64) ** 2))
    return float(np.max(np.abs(got - ref)) / rms)


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def ensure_built():
    """Builds the HIP library if it is not there yet (tests call, never rebuild an existing one)."""
    lib = os.path.join(ROOT, "softmax_learned_covariance_amd", "libparallax.so")
    if not os.path.exists(lib):
        from softmax_learned_covariance_amd import build
        build.build(verbose=False)


def to_pages(kc, vc, page, spare=3, seed=0):
    """Scatter a contiguous cache [B,L,Hkv,d] into a shuffled page pool (storage only) and its table."""
    B, L, Hkv, d = kc.shape
    npb = (L + page - 1) // page
    pad = npb * page - L
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(B * npb + spare, generator=g)[:B * npb].to(kc.device)
    pools = []
    for c in (kc, vc):
        cp = torch.nn.functional.pad(c, (0, 0, 0, 0, 0, pad)) if pad else c
        pool = torch.randn((B * npb + spare, page, Hkv, d), device=kc.device).to(c.dtype)   # junk in spare pages
        pool[perm] = cp.reshape(B * npb, page, Hkv, d)
        pools.append(pool)
    return pools[0], pools[1], perm.reshape(B, npb).to(torch.int32).contiguous()
