"""GPU checks of the output options: bf16 `out` and the correction-to-output ratio.

bf16 out is the fp32 result rounded to nearest even, so it must equal torch's rounding of the fp32
call's output bit for bit (every kernel here is deterministic).  The ratio |out - o| / |out| is
compared with the oracle's out and o (for decode, o is the oracle's decode with P = 0) by the usual
max |err| / rms <= 2e-2, and with the same kernel's own fp32 out and o_sa to 1e-4.
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
    print(f"[outputs] {msg}", flush=True)


def _ratio(out, o):
    num = np.linalg.norm(out - o, axis=-1)
    den = np.linalg.norm(out, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def test_forward_bf16_out_and_ratio(plx):
    _announce("forward: bf16 out, correction ratio")
    w = W.scaled(W.WORKLOADS["layer06"], batch=2, seqlen_q=600, seqlen_k=600)
    q, k, v, P = W.make_inputs(w, device="cuda")
    out32, lse, kbar, o, cor = plx.parallax_attn_fwd(q, k, v, P, window=300, cor=True)
    out16 = plx.parallax_attn_fwd(q, k, v, P, window=300, out_dtype=torch.bfloat16)[0]
    torch.cuda.synchronize()
    assert out16.dtype == torch.bfloat16 and torch.equal(out16, out32.to(torch.bfloat16))
    own = _ratio(host(out32), host(o)).transpose(0, 2, 1)            # [B, Hq, Tq]
    assert np.max(np.abs(host(cor) - own)) <= 1e-4 * max(1.0, np.max(own))
    ref = oracle.fwd(host(q), host(k), host(v), host(P), causal=True, window=300)
    want = _ratio(ref[0], ref[3]).transpose(0, 2, 1)
    assert rel_err(host(cor), want) <= BF16_TOL


def test_probe_bf16_out_and_ratio(plx):
    _announce("probe forward: bf16 out, correction ratio")
    w = W.scaled(W.WORKLOADS["layer06"], batch=2, seqlen_q=500, seqlen_k=700)
    q, k, v, _ = W.make_inputs(w, device="cuda")
    rho = W.make_probe(w, device="cuda")
    out32, lse, o, rk, cor = plx.parallax_attn_fwd_probe(q, k, v, rho, cor=True)
    out16 = plx.parallax_attn_fwd_probe(q, k, v, rho, out_dtype=torch.bfloat16)[0]
    torch.cuda.synchronize()
    assert torch.equal(out16, out32.to(torch.bfloat16))
    ref_out, _, ref_o, _ = oracle.fwd_probe(host(q), host(k), host(v), host(rho), causal=True)
    want = _ratio(ref_out, ref_o).transpose(0, 2, 1)
    assert rel_err(host(cor), want) <= BF16_TOL


def test_decode_bf16_out_and_ratio(plx):
    _announce("decode and paged decode: bf16 out, correction ratio")
    w = W.scaled(W.WORKLOADS["decode"], batch=4, seqlen_k=1200)
    q, kc, vc, P = W.make_inputs(w, device="cuda")
    seqlens = torch.tensor([1200, 1, 0, 640], dtype=torch.int32, device="cuda")
    out32, cor = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, cor=True)
    out16 = plx.parallax_attn_decode(q, kc, vc, P, seqlens=seqlens, out_dtype=torch.bfloat16)
    table = torch.arange(4 * 1200 // 16, dtype=torch.int32, device="cuda").reshape(4, -1)
    kp = kc.reshape(-1, 16, w.heads_kv, w.head_dim)
    vp = vc.reshape(-1, 16, w.heads_kv, w.head_dim)
    pout16, pcor = plx.parallax_attn_decode_paged(q, kp, vp, table, P, seqlens=seqlens, out_dtype=torch.bfloat16,
                                                  cor=True)
    torch.cuda.synchronize()
    assert torch.equal(out16, out32.to(torch.bfloat16))
    assert torch.equal(pout16, out16) and torch.equal(pcor, cor)
    sl = host(seqlens).astype(int)
    ref = oracle.decode(host(q), host(kc), host(vc), host(P), seqlens=sl)
    ref0 = oracle.decode(host(q), host(kc), host(vc), np.zeros(P.shape), seqlens=sl)
    want = _ratio(ref, ref0)
    assert np.all(host(cor)[2] == 0)
    assert rel_err(host(cor), want) <= BF16_TOL
