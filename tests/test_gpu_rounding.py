"""The kernels' errors are the roundings their CPU emulations write out.

The forward and the single-read decode run on inputs drawn on the host; their outputs are compared with
the oracle and with the float64 emulation of each kernel's roundings (the emulations that pin the
fp16-versus-bf16 choice on the CPU).

* Forward, single fp16 operands (split_rows = 0: hi + lo pairs on the first 16 rows only).  A rounding of
  kbar or x moves u, and that decides which way half of U-hat's entries round, so the kernel and the
  emulation draw different rounding errors of one distribution: their rms and largest errors must agree
  within 25% and a factor of two.
* Forward, hi + lo pairs on every row (the default split_rows covers all 256): about 22 significant bits,
  so each row's error stays at fp32's level (below 4e-6 of the row's largest output; measured 2.2e-6 at
  most).  The bound catches pairs formed inconsistently (hi rounded from the fp32 product, lo taken
  against a rounding of the exact product: one fp16 step off wherever the two roundings disagree), which
  reached 5e-6 to 5e-5 here.  The probe form's key gradients are the most exposed to that (1.6e-4 to
  4.6e-4 against 1e-5 with consistent pairs), so they are checked too.
* Single-read decode: u comes from kbar in fp32 and is not rounded, so the kernel's rounding pattern is
  the emulation's and the two outputs lie within a quarter of the emulation's error of each other.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import test_decode_numerics as DN
from tests import test_fwd_numerics as FN
from tests.test_gpu_decode_moment import _Hook
from tests.util import ensure_built, host, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plx():
    ensure_built()
    import softmax_learned_covariance_amd as m
    return m


def _forward(plx, seed, split_rows):
    q, k, v, P = FN._inputs(seed)
    out = plx.parallax_attn_fwd(q.cuda(), k.cuda(), v.cuda(), P.cuda(), causal=True, split_rows=split_rows)[0]
    torch.cuda.synchronize()
    q, k, v, P = (t.to(torch.float64).numpy() for t in (q, k, v, P))
    return host(out)[0], oracle.fwd(q, k, v, P, causal=True)[0][0], (q, k, v, P)


def _rms(x, ref):
    return float(np.sqrt(np.mean((x - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))


@pytest.mark.parametrize("seed", FN.SEEDS)
def test_forward_single_operands_err_as_emulated(plx, seed):
    print(f"[rounding] forward, causal T=256, 2 query heads, split_rows=0, seed {seed}", flush=True)
    got, ref, inputs = _forward(plx, seed, 0)
    emu = FN._emulate_heads(*inputs, FN._f16, split_rows=16)
    mk, me = rel_err(got, ref), rel_err(emu, ref)
    rk, re_ = _rms(got, ref), _rms(emu, ref)
    print(f"[rounding] forward seed {seed}: max err kernel {mk:.2e} emulation {me:.2e}, "
          f"rms err kernel {rk:.2e} emulation {re_:.2e}", flush=True)
    assert 0.8 <= rk / re_ <= 1.25
    assert 0.5 <= mk / me <= 2.0


@pytest.mark.parametrize("seed", FN.SEEDS)
def test_forward_pairs_keep_their_bits(plx, seed):
    print(f"[rounding] forward, causal T=256, 2 query heads, hi + lo on every row, seed {seed}", flush=True)
    got, ref, _ = _forward(plx, seed, -1)
    row = float(np.max(np.abs(got - ref).max(axis=2) / np.abs(ref).max(axis=2)))
    print(f"[rounding] forward pairs seed {seed}: largest row-relative error {row:.2e}", flush=True)
    assert row <= 4e-6


@pytest.mark.parametrize("seed", FN.SEEDS)
def test_probe_backward_pairs_keep_their_bits(plx, seed):
    print(f"[rounding] probe-form backward, causal T=256, hi + lo on every row, seed {seed}", flush=True)
    q, k, v, P, dout = W.make_inputs(FN._workload(), with_dout=True, seed=seed)
    rho = W.make_probe(FN._workload(), seed=seed)
    qc, kc, vc, rc, dc = (t.cuda() for t in (q, k, v, rho, dout))
    out, lse, osa, rk = plx.parallax_attn_fwd_probe(qc, kc, vc, rc, causal=True)
    dk = plx.parallax_attn_bwd_probe(qc, kc, vc, rc, out, dc, lse, osa, rk, causal=True)[1]
    torch.cuda.synchronize()
    ref = oracle.bwd_probe(*(t.to(torch.float64).numpy() for t in (q, k, v, rho, dout)), causal=True)[1]
    err = rel_err(host(dk), ref)
    print(f"[rounding] probe backward pairs seed {seed}: dk {err:.2e}", flush=True)
    assert err <= 3e-5


def test_decode_rounds_as_emulated(plx):
    B, L, Hq, Hkv = 32, 700, 16, 8
    print(f"[rounding] single-read decode, {B} ragged sequences up to {L}, {Hq} / {Hkv} heads", flush=True)
    w = W.scaled(W.WORKLOADS["decode"], batch=B, seqlen_k=L, heads_q=Hq, heads_kv=Hkv)
    q, kc, vc, P = W.make_inputs(w, seed=37)
    rng = np.random.default_rng(37)
    seqlens = [L, 0, 1, 63, 64, 65, 129, L - 1] + rng.integers(1, L + 1, size=B - 8).tolist()
    hook = _Hook(plx, plx.PLX_KERNEL_DECODE_MOMENT)
    try:
        with hook:
            out = plx.parallax_attn_decode(q.cuda(), kc.cuda(), vc.cuda(), P.cuda(),
                                           seqlens=torch.tensor(seqlens, dtype=torch.int32, device="cuda"))
        assert hook.ran(), "the single-read kernel did not run"
    finally:
        hook.close()
    torch.cuda.synchronize()
    got = host(out)
    q, kc, vc, P = (t.to(torch.float64).numpy() for t in (q, kc, vc, P))
    G = Hq // Hkv
    live = [b for b in range(B) if seqlens[b] > 0]
    ref = np.stack([oracle.decode(q[b:b + 1], kc[b:b + 1, :seqlens[b]], vc[b:b + 1, :seqlens[b]], P)[0]
                    for b in live])
    emu = np.stack([np.concatenate([DN._emulate(q[b, g * G:(g + 1) * G], kc[b, :seqlens[b], g],
                                                vc[b, :seqlens[b], g], P[g * G:(g + 1) * G], 128 ** -0.5, DN._f16)
                                    for g in range(Hkv)]) for b in live])
    got = got[live]
    assert np.all(host(out)[[b for b in range(B) if seqlens[b] == 0]] == 0)
    rms = np.sqrt(np.mean(ref ** 2))
    e_kernel, e_emu = rel_err(got, ref), rel_err(emu, ref)
    dist = float(np.max(np.abs(got - emu)) / rms)
    print(f"[rounding] decode: kernel {e_kernel:.2e}, emulation {e_emu:.2e}, apart {dist:.2e}", flush=True)
    assert dist <= 0.25 * e_emu
