"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

from tests.util import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "parallax.h")


@pytest.fixture(scope="module")
def plx():
    ensure_built()
    import softmax_learned_covariance_amd as m
    m.get_lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(parallax_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(plx):
    names = declared_functions()
    assert len(names) == 19, names
    out = subprocess.run(["nm", "-D", "--defined-only", plx.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (parallax_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    # and the binding declares a signature for each of them
    assert sorted(plx.SIGNATURES) == names


def test_abi_version_and_status_strings(plx):
    lib = plx.get_lib()
    hv = int(re.search(r"#define PARALLAX_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.parallax_abi_version() == hv
    for s in range(5):
        assert lib.parallax_status_string(s).startswith(b"PLX_")
    assert lib.parallax_status_string(99) == b"unknown plx_status"


def test_desc_layout_matches_header(plx):
    # 12 int32 fields and one float, no padding
    assert ctypes.sizeof(plx.PlxAttnDesc) == 52


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _desc(plx, **kw):
    base = dict(B=1, Tq=8, Tk=8, Hq=2, Hkv=1, d=16, causal=True, window=0, scale=None,
                dtype=plx.PLX_F32, p_per_query=False, split_rows=-1, out_dtype=plx.PLX_F32)
    base.update(kw)
    return plx.make_desc(base["B"], base["Tq"], base["Tk"], base["Hq"], base["Hkv"], base["d"],
                         base["causal"], base["window"], base["scale"], base["dtype"],
                         base["p_per_query"], base["split_rows"], base["out_dtype"])


def _fwd(plx, desc, q=FAKE, k=FAKE, v=FAKE, P=FAKE, out=FAKE, ws=None, nws=0):
    lib = plx.get_lib()
    return lib.parallax_attn_fwd(ctypes.byref(desc) if desc is not None else None, q, k, v, P, out,
                                 None, None, None, None, ws, nws, None)


def _bwd(plx, desc, ws=FAKE, nws=1 << 40, **null):
    lib = plx.get_lib()
    args = {n: FAKE for n in ("q", "k", "v", "P", "out", "dout", "lse", "kbar", "osa", "dq", "dk", "dv", "dP")}
    args.update(null)
    return lib.parallax_attn_bwd(ctypes.byref(desc), *args.values(), ws, nws, None)


def _dec(plx, desc, q=FAKE, P=FAKE, out=FAKE, ws=FAKE, nws=1 << 40):
    lib = plx.get_lib()
    return lib.parallax_attn_decode(ctypes.byref(desc), q, FAKE, FAKE, None, P, out, None, ws, nws, None)


def test_forward_validation(plx):
    E = plx
    assert _fwd(plx, None) == E.PLX_ERR_INVALID
    assert b"NULL" in plx.get_lib().parallax_last_error()
    assert _fwd(plx, _desc(plx, Hq=3, Hkv=2)) == E.PLX_ERR_INVALID
    assert _fwd(plx, _desc(plx, B=-1)) == E.PLX_ERR_INVALID
    assert _fwd(plx, _desc(plx, Hkv=0)) == E.PLX_ERR_INVALID
    assert _fwd(plx, _desc(plx, d=0)) == E.PLX_ERR_INVALID
    assert _fwd(plx, _desc(plx, d=129)) == E.PLX_ERR_UNSUPPORTED
    assert _fwd(plx, _desc(plx, dtype=7)) == E.PLX_ERR_INVALID
    assert _fwd(plx, _desc(plx, scale=float("nan"))) == E.PLX_ERR_INVALID
    assert _fwd(plx, _desc(plx), q=None) == E.PLX_ERR_INVALID
    assert _fwd(plx, _desc(plx), out=None) == E.PLX_ERR_INVALID
    assert _fwd(plx, _desc(plx), k=None) == E.PLX_ERR_INVALID
    # empty problems are valid and launch nothing
    assert _fwd(plx, _desc(plx, B=0)) == E.PLX_OK
    assert _fwd(plx, _desc(plx, Tq=0), q=None, out=None) == E.PLX_OK
    assert plx.get_lib().parallax_last_error() == b""


def test_workspace_queries(plx):
    lib = plx.get_lib()
    assert lib.parallax_attn_fwd_workspace(None) == 0
    assert lib.parallax_attn_bwd_workspace(ctypes.byref(_desc(plx))) > 0
    assert lib.parallax_attn_bwd_workspace(ctypes.byref(_desc(plx, Hq=3, Hkv=2))) == 0
    assert lib.parallax_attn_decode_workspace(ctypes.byref(_desc(plx, Tq=2))) == 0


def test_backward_validation(plx):
    E = plx
    d = _desc(plx)
    need = plx.get_lib().parallax_attn_bwd_workspace(ctypes.byref(d))
    assert _bwd(plx, d, nws=need - 1) == E.PLX_ERR_WORKSPACE
    assert b"workspace" in plx.get_lib().parallax_last_error()
    assert _bwd(plx, d, ws=None, nws=need) == E.PLX_ERR_INVALID
    assert _bwd(plx, _desc(plx, p_per_query=True)) == E.PLX_ERR_UNSUPPORTED
    assert _bwd(plx, d, lse=None) == E.PLX_ERR_INVALID
    assert _bwd(plx, d, dP=None) == E.PLX_ERR_INVALID
    assert _bwd(plx, d, dk=None) == E.PLX_ERR_INVALID


def test_decode_validation(plx):
    E = plx
    assert _dec(plx, _desc(plx, Tq=0)) == E.PLX_ERR_INVALID
    assert _dec(plx, _desc(plx, Tq=2)) == E.PLX_ERR_UNSUPPORTED     # several new tokens: bf16 fast path only
    assert _dec(plx, _desc(plx, Tq=1, p_per_query=True)) == E.PLX_ERR_UNSUPPORTED
    assert _dec(plx, _desc(plx, Tq=1), q=None) == E.PLX_ERR_INVALID
    assert _dec(plx, _desc(plx, Tq=1, B=0)) == E.PLX_OK


def _probe(plx, desc, q=FAKE, rho=FAKE, out=FAKE, ws=FAKE, nws=1 << 40):
    lib = plx.get_lib()
    return lib.parallax_attn_fwd_probe(ctypes.byref(desc), q, FAKE, FAKE, rho, out, None, None, None, None, ws, nws,
                                       None)


def test_probe_validation(plx):
    E = plx
    lib = plx.get_lib()
    bf = dict(dtype=plx.PLX_BF16, d=128)
    assert _probe(plx, _desc(plx)) == E.PLX_ERR_UNSUPPORTED             # fp32
    assert _probe(plx, _desc(plx, dtype=plx.PLX_BF16)) == E.PLX_ERR_UNSUPPORTED   # head_dim 16
    assert _probe(plx, _desc(plx, Hq=3, Hkv=1, **bf)) == E.PLX_ERR_UNSUPPORTED    # 3 heads per group
    assert _probe(plx, _desc(plx, Hq=3, Hkv=2, **bf)) == E.PLX_ERR_INVALID
    d = _desc(plx, **bf)
    need = lib.parallax_attn_fwd_probe_workspace(ctypes.byref(d))
    assert need > 0
    assert lib.parallax_attn_fwd_probe_workspace(ctypes.byref(_desc(plx))) == 0
    assert _probe(plx, d, nws=need - 1) == E.PLX_ERR_WORKSPACE
    assert _probe(plx, d, ws=None, nws=need) == E.PLX_ERR_INVALID
    assert _probe(plx, d, rho=None) == E.PLX_ERR_INVALID
    assert b"rho" in lib.parallax_last_error()
    assert _probe(plx, d, out=None) == E.PLX_ERR_INVALID
    assert _probe(plx, _desc(plx, B=0, **bf)) == E.PLX_OK


def test_probe_backward_validation(plx):
    E = plx
    lib = plx.get_lib()
    bf = dict(dtype=plx.PLX_BF16, d=128)

    def call(desc, ws=FAKE, nws=1 << 40, **null):
        args = {n: FAKE for n in ("q", "k", "v", "rho", "out", "dout", "lse", "osa", "rk", "dq", "dk", "dv", "drho")}
        args.update(null)
        return lib.parallax_attn_bwd_probe(ctypes.byref(desc), *args.values(), ws, nws, None)

    assert call(_desc(plx)) == E.PLX_ERR_UNSUPPORTED                      # fp32
    assert call(_desc(plx, Hq=3, Hkv=1, **bf)) == E.PLX_ERR_UNSUPPORTED   # 3 query heads per group
    d = _desc(plx, **bf)
    need = lib.parallax_attn_bwd_probe_workspace(ctypes.byref(d))
    assert need > 0
    assert call(d, nws=need - 1) == E.PLX_ERR_WORKSPACE
    assert call(d, ws=None, nws=need) == E.PLX_ERR_INVALID
    for name in ("rho", "rk", "osa", "drho", "dk"):
        assert call(d, **{name: None}) == E.PLX_ERR_INVALID, name
    assert call(_desc(plx, B=0, **bf)) == E.PLX_OK
    assert lib.parallax_attn_bwd_probe_workspace(ctypes.byref(_desc(plx, B=0, **bf))) == 0


def test_paged_decode_validation(plx):
    E = plx
    lib = plx.get_lib()
    bf = dict(dtype=plx.PLX_BF16, d=128, Tq=1)

    def call(desc, num_pages=4, page=16, table=FAKE, q=FAKE, ws=FAKE, nws=1 << 40, stride=None):
        if stride is None:
            stride = (desc.seqlen_k + page - 1) // page if page > 0 else 1
        return lib.parallax_attn_decode_paged(ctypes.byref(desc), q, FAKE, FAKE, num_pages, page, table, stride,
                                              None, FAKE, FAKE, None, ws, nws, None)

    d = _desc(plx, **bf)
    assert call(_desc(plx, dtype=plx.PLX_BF16, d=128, Tq=0)) == E.PLX_ERR_INVALID
    for page in (0, 3, 48, 1 << 17):
        assert call(d, page=page) == E.PLX_ERR_INVALID, page
    assert b"page_size" in lib.parallax_last_error()
    assert call(d, num_pages=0) == E.PLX_ERR_INVALID
    # the table's row stride must cover seqlen_k; a wider table (sized for the cache's capacity) is fine
    pages = (d.seqlen_k + 15) // 16
    assert call(d, stride=pages - 1) == E.PLX_ERR_INVALID
    assert b"block_table_stride" in lib.parallax_last_error()
    assert call(d, stride=pages + 7, nws=0) == E.PLX_ERR_WORKSPACE     # passed the stride check
    assert call(_desc(plx, Tq=1)) == E.PLX_ERR_UNSUPPORTED                       # fp32
    assert call(_desc(plx, Hq=3, Hkv=1, **bf)) == E.PLX_ERR_UNSUPPORTED          # 3 query heads per group
    assert call(d, table=None) == E.PLX_ERR_INVALID
    assert call(d, q=None) == E.PLX_ERR_INVALID
    need = lib.parallax_attn_decode_paged_workspace(ctypes.byref(d))
    assert need > 0 and need == lib.parallax_attn_decode_workspace(ctypes.byref(d))
    assert call(d, nws=need - 1) == E.PLX_ERR_WORKSPACE
    assert call(_desc(plx, B=0, **bf), ws=None, nws=0) in (E.PLX_OK, E.PLX_ERR_INVALID)


def test_noalloc_decode_validation(plx):
    """The no-allocation decode validates like the workspace decode and refuses a decode whose scratch
    exceeds its fixed array -- before any HIP call, so this runs without a GPU."""
    E = plx
    lib = plx.get_lib()
    cap = lib.parallax_attn_decode_noalloc_max_scratch()
    assert cap == 64 << 20

    def call(desc, q=FAKE):
        return lib.parallax_attn_decode_noalloc(ctypes.byref(desc), q, FAKE, FAKE, None, FAKE, FAKE, None, None)

    big = _desc(plx, B=4096, Tq=8, Tk=32768, Hq=16, Hkv=8, d=128, dtype=plx.PLX_BF16)
    assert lib.parallax_attn_decode_workspace(ctypes.byref(big)) > cap
    assert call(big) == E.PLX_ERR_WORKSPACE
    assert b"scratch" in lib.parallax_last_error()
    assert call(_desc(plx, dtype=plx.PLX_BF16, d=128, Tq=0)) == E.PLX_ERR_INVALID
    assert call(_desc(plx, Tq=3)) == E.PLX_ERR_UNSUPPORTED            # several tokens on the fp32 path
    assert call(_desc(plx, dtype=plx.PLX_BF16, d=128, Tq=1), q=None) == E.PLX_ERR_INVALID
    assert call(_desc(plx, B=0, dtype=plx.PLX_BF16, d=128, Tq=1)) == E.PLX_OK


def test_output_options_validation(plx):
    """out_dtype must be a known dtype; bf16 out and the correction ratio need the bf16 fast path; the
    backwards read an fp32 out."""
    E = plx
    lib = plx.get_lib()
    assert _fwd(plx, _desc(plx, out_dtype=7)) == E.PLX_ERR_INVALID
    assert b"out_dtype" in lib.parallax_last_error()
    assert _fwd(plx, _desc(plx, out_dtype=plx.PLX_BF16)) == E.PLX_ERR_UNSUPPORTED     # fp32 inputs
    d = _desc(plx)
    assert lib.parallax_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None, 0,
                                 None) == E.PLX_ERR_UNSUPPORTED                          # cor on the fp32 path
    assert _dec(plx, _desc(plx, Tq=1, out_dtype=plx.PLX_BF16)) == E.PLX_ERR_UNSUPPORTED
    bfd = _desc(plx, dtype=plx.PLX_BF16, d=128, out_dtype=plx.PLX_BF16)
    assert _bwd(plx, bfd) == E.PLX_ERR_UNSUPPORTED
    assert b"fp32 out" in lib.parallax_last_error()


def test_bench_refuses_more_than_one_gpu():
    """The library has no multi-GPU path: bench.py --gpus 2 stops with a message before touching a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_summary_rows_parse():
    """Every kernel row of the committed HBM-traffic summary has the six fields bench.py reads (name,
    kernel, FETCH KiB, WRITE KiB, bytes, source hash), so no stored figure is silently dropped."""
    path = os.path.join(ROOT, "profiles", "traffic_layer17_decode.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#") and not ln.startswith("name")]
    assert rows
    for f in rows:
        assert len(f) == 6, f
        float(f[2]), float(f[3]), float(f[4])
        assert len(f[5]) == 16


def test_decode_path_selection(plx):
    """The process-wide decode path accepts its two values only (no GPU call is made)."""
    lib = plx.get_lib()
    for bad in (2, -1, 99):
        assert lib.parallax_set_decode_path(bad) == plx.PLX_ERR_INVALID
        assert b"decode_path" in lib.parallax_last_error()
    assert lib.parallax_set_decode_path(plx.PLX_DECODE_TWO_PASS) == plx.PLX_OK
    assert lib.parallax_set_decode_path(plx.PLX_DECODE_AUTO) == plx.PLX_OK
