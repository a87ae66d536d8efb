"""Benchmark of the Parallax attention operator on one MI355X.

A step is one forward plus one backward of the 1.7B-like layer (B=2, T=8192,
16 query / 8 key-value heads, d=128, bf16 inputs, causal) on synthetic seeded
inputs already resident in HBM.  `value` is the algorithmic TFLOP/s of the step
(forward 12d flop per visible pair + 2d^2 per row, backward 24d per pair + 4d^2
per row; the fp32 early-row path and precision splits are not counted).  The
decode workload (64 queries against a 32768-long cache) is timed after the
steps and reported in its own object.  One JSON line goes to stdout; progress
goes to stderr.

The probe-form forward (caller-supplied probe rho, one pass) and a probe-form
forward + backward step are timed on the same layer shape after the steps and
reported in their own object too.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--no-probe]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Parallax attn fwd/bwd TFLOP/s + tokens/s at T=8192,d=128 bf16; % MFMA peak"
PEAK_F16_TFLOPS = 2516.6     # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs_rows(w, row_begin=0):
    """(pairs, rows) over batch and query heads for query rows >= row_begin."""
    off = w.seqlen_k - w.seqlen_q
    pairs = 0
    for i in range(row_begin, w.seqlen_q):
        hi = min(w.seqlen_k, i + off + 1) if w.causal else w.seqlen_k
        lo = max(0, i + off - w.window + 1) if w.window > 0 else 0
        pairs += max(0, hi - lo)
    nbh = w.batch * w.heads_q
    return pairs * nbh, max(0, w.seqlen_q - row_begin) * nbh


def fwd_flops(w, row_begin=0):
    """Forward: 12d per visible pair (pass 1 QK^T 2d + p[V|K] 4d, pass 2 QK^T 2d + UK^T 2d + WV 2d) + 2d^2 per row (u)."""
    pairs, rows = visible_pairs_rows(w, row_begin)
    return 12 * w.head_dim * pairs + 2 * w.head_dim ** 2 * rows


def probe_flops(w, row_begin=0):
    """Probe-form forward: 8d per visible pair (Q K^T, rho K^T, p V and (p r) V)."""
    pairs, _ = visible_pairs_rows(w, row_begin)
    return 8 * w.head_dim * pairs


def probe_bwd_flops(w, row_begin=0):
    """Probe-form backward: 24d per visible pair (no projector terms)."""
    pairs, _ = visible_pairs_rows(w, row_begin)
    return 24 * w.head_dim * pairs


def bwd_flops(w, row_begin=0):
    """Backward: 24d per visible pair + 4d^2 per row (P du and the dP outer product)."""
    pairs, rows = visible_pairs_rows(w, row_begin)
    return 24 * w.head_dim * pairs + 4 * w.head_dim ** 2 * rows


def bwd_rows_flops(w, row_begin=0):
    """Algorithmic share of the query-major backward kernel: du (S, G, (pG)K: 6d per pair) and
    P du (2d^2 per row); its recomputation of u = P^T (q - kbar) is not counted."""
    pairs, rows = visible_pairs_rows(w, row_begin)
    return 6 * w.head_dim * pairs + 2 * w.head_dim ** 2 * rows


def bwd_dq_flops(w, row_begin=0):
    """dq kernel: scale * ds K (2d per pair) from the stored ds."""
    pairs, _ = visible_pairs_rows(w, row_begin)
    return 2 * w.head_dim * pairs


def bwd_keys_flops(w, row_begin=0):
    """Key-major backward kernel: S, T, E, G (8d), dv (2d) and dk (6d) per visible pair."""
    pairs, _ = visible_pairs_rows(w, row_begin)
    return 16 * w.head_dim * pairs


# Source files of each timed kernel: a stored traffic figure is used only while they are unchanged.
KERNEL_SOURCES = {"fwd": ["fast_fwd.hip", "fast_common.h"], "bwd_rows": ["fast_bwd.hip", "fast_common.h"],
                  "bwd_keys": ["fast_bwd.hip", "fast_common.h"], "bwd_dq": ["fast_bwd.hip", "fast_common.h"],
                  "decode_pass1": ["fast_decode.hip", "fast_common.h"],
                  "decode_pass2": ["fast_decode.hip", "fast_common.h"],
                  "decode_moment": ["fast_decode_moment.hip", "fast_common.h"],
                  "probe": ["fast_fwd.hip", "fast_common.h"]}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_layer17_decode.txt")


def source_hash(name):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "softmax_learned_covariance_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch of kernel `name` from the committed FETCH_SIZE/WRITE_SIZE summary
    (copy-calibrated), or None when the summary is missing or the kernel's sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                f = line.split()
                if len(f) == 6 and f[0] == name:
                    return float(f[4]) if f[5] == source_hash(name) else None
    except OSError:
        pass
    return None


class HipEvents:
    """Thin ctypes access to HIP events (timing on the library's stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w):
    """The oracle (numpy, float64 as in every parity test, and its float32 timing mode) timed on this
    host on a bounded sample of the workload.

    Sample: batch entry 0 (all query heads, all T rows), forward + backward; scaled to TFLOP/s with the
    same algorithmic count as the GPU figures.
    """
    import numpy as np
    import torch
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    ws = W.scaled(w, batch=1)
    q, k, v, P, dout = W.make_inputs(ws, device="cpu", with_dout=True)
    h = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    fl = fwd_flops(ws) + bwd_flops(ws)
    t0 = time.perf_counter()
    oracle.fwd(h(q), h(k), h(v), h(P), causal=True)
    oracle.bwd(h(q), h(k), h(v), h(P), h(dout), causal=True)
    dt = time.perf_counter() - t0
    # the float32 mode on half the heads (8 query, 4 key/value heads), to keep the host time bounded
    w32 = W.scaled(ws, heads_q=max(1, ws.heads_q // 2), heads_kv=max(1, ws.heads_kv // 2))
    q, k, v, P, dout = W.make_inputs(w32, device="cpu", with_dout=True)
    fl32 = fwd_flops(w32) + bwd_flops(w32)
    with oracle.precision(np.float32):
        t0 = time.perf_counter()
        oracle.fwd(h(q), h(k), h(v), h(P), causal=True)
        oracle.bwd(h(q), h(k), h(v), h(P), h(dout), causal=True)
        dt32 = time.perf_counter() - t0
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"numpy float64 oracle, forward+backward of batch entry 0 (all {ws.heads_q} query heads), "
                      f"all {ws.seqlen_q} rows of the {w.name} workload: {fl / 1e9:.1f} GFLOP in {dt:.1f} s",
            "seconds": round(dt, 2),
            "fp32": {"value": round(fl32 / dt32 / 1e12, 6), "unit": "TFLOP/s", "seconds": round(dt32, 2),
                     "sample": f"the same oracle in its float32 timing mode, batch entry 0 with {w32.heads_q} query "
                               f"and {w32.heads_kv} key/value heads: {fl32 / 1e9:.1f} GFLOP"},
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(), "blas_threads": int(threads)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="layer17")
    ap.add_argument("--split-rows", type=int, default=-1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the decode batch/context sweep")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the layer06 forward and train06 training-step objects")
    ap.add_argument("--probe-only", action="store_true",
                    help="time only the probe form (a profiling run that separates its kernels from the "
                         "projector form's, which share kernel names)")
    ap.add_argument("--samples", type=int, default=12,
                    help="extra kernel-event samples per backward kernel (beyond the timed steps)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy, the reference for HBM traffic counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Parallax operator here is a single-GPU kernel "
              "library with no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if not os.path.exists(os.path.join(ROOT, "softmax_learned_covariance_amd", "libparallax.so")):
        from softmax_learned_covariance_amd import build as b
        b.build()
    import torch
    import softmax_learned_covariance_amd as plx
    import workloads as W

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")
        del src, dst
    w = W.WORKLOADS[args.workload]
    log(f"workload {w}")
    q, k, v, P, dout = W.make_inputs(w, device=dev, with_dout=True)
    torch.cuda.synchronize()
    lib = plx.get_lib()
    ev = HipEvents()
    split = args.split_rows

    # the fast path leaves rows < split_rows to its hi/lo-split kernels
    fast = w.dtype == "bf16" and w.head_dim == 128
    r0 = (256 if split < 0 else split) if fast else 0
    r0 = min(r0, w.seqlen_q)
    def kernel_samples(call, kid, n):
        """n calls of `call` with the event hook on kernel `kid`: that kernel's launch times (ms)."""
        pairs = [(ev.create(), ev.create()) for _ in range(n)]
        for e in pairs:
            lib.parallax_set_kernel_events(kid, *e)
            call()
        lib.parallax_set_kernel_events(0, None, None)
        torch.cuda.synchronize()
        return [ev.elapsed_ms(a, b) for a, b in pairs]

    bwd_cycle = (("bwd_rows", plx.PLX_KERNEL_BWD_ROWS), ("bwd_keys", plx.PLX_KERNEL_BWD_KEYS),
                 ("bwd_dq", plx.PLX_KERNEL_BWD_DQ))
    K = args.steps
    if args.probe_only:
        result = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1,
                  "note": "probe form only (a profiling run)"}
    else:
        def step():
            out, lse, kbar, o = plx.parallax_attn_fwd(q, k, v, P, split_rows=split)
            plx.parallax_attn_bwd(q, k, v, P, out, dout, lse, kbar, o, split_rows=split)

        for i in range(args.warmup):
            step()
            torch.cuda.synchronize()
            log(f"warmup step {i + 1}/{args.warmup} done")

        # Timed region: K steps.  The kernel-event hook brackets one kernel per library call: every
        # step times the forward kernel, and the backward cycles through its three main kernels.
        evs = {n: [] for n in ("fwd", "bwd_rows", "bwd_keys", "bwd_dq")}
        pool = [(ev.create(), ev.create()) for _ in range(2 * K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            e_f = pool[2 * i]
            lib.parallax_set_kernel_events(plx.PLX_KERNEL_FWD, *e_f)
            out, lse, kbar, o = plx.parallax_attn_fwd(q, k, v, P, split_rows=split)
            which, kid = bwd_cycle[i % 3]
            e_b = pool[2 * i + 1]
            lib.parallax_set_kernel_events(kid, *e_b)
            plx.parallax_attn_bwd(q, k, v, P, out, dout, lse, kbar, o, split_rows=split)
            evs["fwd"].append(e_f)
            evs[which].append(e_b)
        lib.parallax_set_kernel_events(0, None, None)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        log(f"timed {K} steps in {elapsed:.3f} s")

        # more samples of each backward kernel, outside the timed region
        extra = {}
        for which, kid in bwd_cycle:
            extra[which] = kernel_samples(
                lambda: plx.parallax_attn_bwd(q, k, v, P, out, dout, lse, kbar, o, split_rows=split), kid, args.samples)

        kern = {}
        for n, flops_fn in (("fwd", fwd_flops), ("bwd_rows", bwd_rows_flops), ("bwd_keys", bwd_keys_flops),
                            ("bwd_dq", bwd_dq_flops)):
            if not evs[n]:
                continue
            ms = sorted([ev.elapsed_ms(a, b) for a, b in evs[n]] + extra.get(n, []))
            avg = sum(ms) / len(ms)
            fl = flops_fn(w, r0)
            kern[n] = {"avg_ms": round(avg, 4), "median_ms": round(ms[len(ms) // 2], 4), "launches": len(ms),
                       "algorithmic_flop": fl, "tflops": round(fl / (avg * 1e-3) / 1e12, 3),
                       "frac_of_peak": round(fl / (avg * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)}
        ms_step = elapsed / K * 1e3
        step_flops = fwd_flops(w) + bwd_flops(w)
        value = step_flops / (ms_step * 1e-3) / 1e12
        dom = max(kern, key=lambda n: kern[n]["avg_ms"])
        dk = kern[dom]
        tr = measured_traffic(dom)
        roofline = {"bound": "mfma", "achieved": dk["tflops"], "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(dk["tflops"] / PEAK_F16_TFLOPS, 4), "traffic": None if tr is None else round(tr),
                    "traffic_unit": "bytes per launch (HBM, FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
                    "kernel": dom, "avg_ms": dk["avg_ms"], "algorithmic_flop_per_launch": dk["algorithmic_flop"]}
        result = {
            "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16",
            "data": "synthetic (seeded N(0,1) inputs rounded to bf16, K rows normed to sqrt(d), P ~ N(0, 0.02^2))",
            "config": {"workload": f"{w.name}: Parallax layer forward+backward, B={w.batch}, T={w.seqlen_q}, "
                                   f"Hq={w.heads_q}, Hkv={w.heads_kv}, d={w.head_dim}, causal, bf16 inputs, fp32 outputs",
                       "global_batch": w.batch, "seq_len": w.seqlen_q, "parallelism": "single GPU",
                       "split_rows": r0},
            "tokens_per_s": round(w.batch * w.seqlen_q / (ms_step * 1e-3), 1),
            "kernels": kern,
            "roofline": roofline,
        }

    if not args.no_probe:
        log("probe-form forward")
        rho = W.make_probe(w, device=dev)
        for _ in range(2):
            plx.parallax_attn_fwd_probe(q, k, v, rho, split_rows=split)
        torch.cuda.synchronize()
        Kp = max(6, K)
        pev = [(ev.create(), ev.create()) for _ in range(Kp)]
        t0 = time.perf_counter()
        for i in range(Kp):
            lib.parallax_set_kernel_events(plx.PLX_KERNEL_FWD_PROBE, *pev[i])
            plx.parallax_attn_fwd_probe(q, k, v, rho, split_rows=split)
        lib.parallax_set_kernel_events(0, None, None)
        torch.cuda.synchronize()
        dtp = (time.perf_counter() - t0) / Kp
        pms = sorted(ev.elapsed_ms(a, b) for a, b in pev)
        pavg = sum(pms) / len(pms)
        pfl = probe_flops(w, r0)
        ptf = pfl / (pavg * 1e-3) / 1e12
        result["probe"] = {
            "workload": f"{w.name} probe-form forward: B={w.batch}, T={w.seqlen_q}, Hq={w.heads_q}, "
                        f"Hkv={w.heads_kv}, d={w.head_dim}, causal, bf16 inputs, rho ~ N(0, (0.02 sqrt(d))^2)",
            "ms_per_call": round(dtp * 1e3, 4),
            "tflops_per_call": round(probe_flops(w) / dtp / 1e12, 3),
            "kernel": {"avg_ms": round(pavg, 4), "median_ms": round(pms[len(pms) // 2], 4), "launches": len(pms),
                       "algorithmic_flop": pfl, "tflops": round(ptf, 3),
                       "frac_of_peak": round(ptf / PEAK_F16_TFLOPS, 4)},
            "roofline": {"bound": "mfma", "achieved": round(ptf, 3), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ptf / PEAK_F16_TFLOPS, 4),
                         "traffic": None if measured_traffic("probe") is None else round(measured_traffic("probe"))}}
        log(f"probe forward {dtp * 1e3:.3f} ms/call, kernel {pavg:.3f} ms ({ptf:.0f} TFLOP/s)")

        def probe_step():
            f = plx.parallax_attn_fwd_probe(q, k, v, rho, split_rows=split)
            plx.parallax_attn_bwd_probe(q, k, v, rho, f[0], dout, *f[1:], split_rows=split)

        probe_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(Kp):
            probe_step()
        torch.cuda.synchronize()
        dts = (time.perf_counter() - t0) / Kp
        sfl = probe_flops(w) + probe_bwd_flops(w)
        result["probe"]["step"] = {"what": "probe-form forward + backward (dq, dk, dv, drho)",
                                   "ms_per_step": round(dts * 1e3, 4), "tflops": round(sfl / dts / 1e12, 3),
                                   "algorithmic_flop": sfl, "steps": Kp}
        log(f"probe step {dts * 1e3:.3f} ms ({sfl / dts / 1e12:.0f} TFLOP/s)")
        del rho

    if not args.no_configs:
        result["configs"] = {}
        # layer06 (0.6B-like layer) forward
        w2 = W.WORKLOADS["layer06"]
        log(f"config {w2.name} forward")
        q2, k2, v2, P2 = W.make_inputs(w2, device=dev)
        fwd2 = lambda: plx.parallax_attn_fwd(q2, k2, v2, P2, split_rows=split)  # noqa: E731
        for _ in range(2):
            fwd2()
        torch.cuda.synchronize()
        n2 = max(10, K)
        t0 = time.perf_counter()
        for _ in range(n2):
            fwd2()
        torch.cuda.synchronize()
        dt2c = (time.perf_counter() - t0) / n2
        ks2 = kernel_samples(fwd2, plx.PLX_KERNEL_FWD, n2)
        r2 = min(r0, w2.seqlen_q)
        kfl = fwd_flops(w2, r2)
        kavg = sum(ks2) / len(ks2)
        result["configs"]["layer06_fwd"] = {
            "workload": f"{w2.name}: forward, B={w2.batch}, T={w2.seqlen_q}, Hq={w2.heads_q}, Hkv={w2.heads_kv}, "
                        f"d={w2.head_dim}, causal, bf16",
            "ms_per_call": round(dt2c * 1e3, 4), "tflops": round(fwd_flops(w2) / dt2c / 1e12, 3),
            "tokens_per_s": round(w2.batch * w2.seqlen_q / dt2c, 1),
            "roofline": {"bound": "mfma", "kernel": "fwd", "avg_ms": round(kavg, 4), "launches": len(ks2),
                         "achieved": round(kfl / (kavg * 1e-3) / 1e12, 3), "peak": PEAK_F16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(kfl / (kavg * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
                         "algorithmic_flop_per_launch": kfl}}
        log(f"layer06 forward {dt2c * 1e3:.3f} ms/call, kernel {kavg:.3f} ms")
        del q2, k2, v2, P2

        def train_step_object(w4):
            """Forward + backward of workload w4: the step time and each main kernel's average launch."""
            q4_, k4_, v4_, P4_, d4_ = W.make_inputs(w4, device=dev, with_dout=True)
            f4 = plx.parallax_attn_fwd(q4_, k4_, v4_, P4_, split_rows=split)

            def step4():
                f = plx.parallax_attn_fwd(q4_, k4_, v4_, P4_, split_rows=split)
                plx.parallax_attn_bwd(q4_, k4_, v4_, P4_, f[0], d4_, *f[1:], split_rows=split)

            step4()
            torch.cuda.synchronize()
            n4 = max(6, K)
            t0 = time.perf_counter()
            for _ in range(n4):
                step4()
            torch.cuda.synchronize()
            dt4c = (time.perf_counter() - t0) / n4
            r4 = min(r0, w4.seqlen_q)
            k4 = {}
            calls = {"fwd": (lambda: plx.parallax_attn_fwd(q4_, k4_, v4_, P4_, split_rows=split), plx.PLX_KERNEL_FWD,
                             fwd_flops)}
            bcall = lambda: plx.parallax_attn_bwd(q4_, k4_, v4_, P4_, f4[0], d4_, *f4[1:], split_rows=split)  # noqa: E731
            for n_, kid in bwd_cycle:
                calls[n_] = (bcall, kid, {"bwd_rows": bwd_rows_flops, "bwd_keys": bwd_keys_flops,
                                          "bwd_dq": bwd_dq_flops}[n_])
            for n_, (call, kid, ffn) in calls.items():
                ms_ = kernel_samples(call, kid, max(8, args.samples))
                avg = sum(ms_) / len(ms_)
                fl_ = ffn(w4, r4)
                k4[n_] = {"avg_ms": round(avg, 4), "launches": len(ms_), "algorithmic_flop": fl_,
                          "tflops": round(fl_ / (avg * 1e-3) / 1e12, 3),
                          "frac_of_peak": round(fl_ / (avg * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4)}
            dom4 = max(k4, key=lambda n_: k4[n_]["avg_ms"])
            sfl4 = fwd_flops(w4) + bwd_flops(w4)
            obj = {
                "workload": f"{w4.name}: forward + backward, B={w4.batch}, T={w4.seqlen_q}, Hq={w4.heads_q}, "
                            f"Hkv={w4.heads_kv}, d={w4.head_dim}, causal, bf16 (flops counted at d={w4.head_dim})",
                "ms_per_step": round(dt4c * 1e3, 4), "tflops": round(sfl4 / dt4c / 1e12, 3),
                "tokens_per_s": round(w4.batch * w4.seqlen_q / dt4c, 1), "kernels": k4,
                "roofline": {"bound": "mfma", "kernel": dom4, "avg_ms": k4[dom4]["avg_ms"],
                             "achieved": k4[dom4]["tflops"], "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                             "frac": k4[dom4]["frac_of_peak"],
                             "algorithmic_flop_per_launch": k4[dom4]["algorithmic_flop"]}}
            log(f"{w4.name} d={w4.head_dim} step {dt4c * 1e3:.3f} ms ({sfl4 / dt4c / 1e12:.0f} TFLOP/s); "
                + ", ".join(f"{n_} {k4[n_]['avg_ms']:.3f} ms ({k4[n_]['frac_of_peak']:.3f})" for n_ in k4))
            del q4_, k4_, v4_, P4_, d4_, f4
            torch.cuda.empty_cache()
            return obj

        # layer17's shape at head dim 64 (the pages' compute-matched control: smaller heads): forward + backward
        log("config layer17 at head dim 64, training step")
        result["configs"]["layer17_d64_step"] = train_step_object(W.scaled(W.WORKLOADS["layer17"], head_dim=64))
        # train06 (0.6B-like training step): forward + backward
        log("config train06 training step")
        result["configs"]["train06_step"] = train_step_object(W.WORKLOADS["train06"])

    if not args.no_decode:
        wd = W.WORKLOADS["decode"]
        log("decode workload")
        del q, k, v, P, dout
        torch.cuda.empty_cache()
        qd, kc, vc, Pd = W.make_inputs(wd, device=dev)
        for _ in range(2):
            plx.parallax_attn_decode(qd, kc, vc, Pd)
        torch.cuda.synchronize()
        Kd = max(6, K)
        cache_bytes = 2 * wd.batch * wd.seqlen_k * wd.heads_kv * wd.head_dim * 2
        other = (wd.batch * wd.heads_q * wd.head_dim) * (2 + 4) + wd.heads_q * wd.head_dim ** 2 * 2
        alg = cache_bytes + other
        keys = wd.batch * wd.seqlen_k * wd.heads_q   # (key, query head) pairs
        # the default path (the single-read kernel for this shape), timed with its kernel's events
        dev_ev = [(ev.create(), ev.create()) for _ in range(Kd)]
        t0 = time.perf_counter()
        for i in range(Kd):
            lib.parallax_set_kernel_events(plx.PLX_KERNEL_DECODE_MOMENT, *dev_ev[i])
            plx.parallax_attn_decode(qd, kc, vc, Pd)
        lib.parallax_set_kernel_events(0, None, None)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / Kd
        kms_m = sum(ev.elapsed_ms(a, b) for a, b in dev_ev) / Kd
        # the two-pass kernels on the same inputs (pass 1 and pass 2 events on alternate calls)
        plx.parallax_set_decode_path(plx.PLX_DECODE_TWO_PASS)
        for _ in range(2):
            plx.parallax_attn_decode(qd, kc, vc, Pd)
        torch.cuda.synchronize()
        dev_ev2 = [(ev.create(), ev.create()) for _ in range(Kd)]
        t0 = time.perf_counter()
        for i in range(Kd):
            lib.parallax_set_kernel_events(plx.PLX_KERNEL_DECODE_PASS1 if i % 2 == 0 else plx.PLX_KERNEL_DECODE_PASS2,
                                           *dev_ev2[i])
            plx.parallax_attn_decode(qd, kc, vc, Pd)
        lib.parallax_set_kernel_events(0, None, None)
        torch.cuda.synchronize()
        dt2 = (time.perf_counter() - t0) / Kd
        plx.parallax_set_decode_path(plx.PLX_DECODE_AUTO)
        p1 = [ev.elapsed_ms(a, b) for a, b in dev_ev2[0::2]]
        p2 = [ev.elapsed_ms(a, b) for a, b in dev_ev2[1::2]]
        kms1, kms2 = sum(p1) / len(p1), sum(p2) / len(p2)
        t1, t2 = measured_traffic("decode_pass1"), measured_traffic("decode_pass2")
        gbs = alg / (kms_m * 1e-3) / 1e9
        # matrix-core work of the single-read kernel as executed: per (key, query head) the moment's 2 d^2
        # and kbar~ (a 32-row ones operand against y: 64 d); per key and kv head o~ (32 weight rows against
        # the values: 64 d) and the scores (16 padded columns: 32 d)
        d = wd.head_dim
        G = wd.heads_q // wd.heads_kv
        mfma_flop = keys * (2 * d * d + 64 * d) + keys // G * (64 * d + 32 * d)
        result["decode"] = {
            "workload": f"decode: B={wd.batch} new queries, cache L={wd.seqlen_k}, Hq={wd.heads_q}, "
                        f"Hkv={wd.heads_kv}, d={wd.head_dim}, bf16",
            "path": "single-read (one pass over the cache, key/value moment on MFMA)",
            "ms_per_call": round(dt * 1e3, 4), "tokens_per_s": round(wd.batch / dt, 1),
            "kernels": {"single_read": {"avg_ms": round(kms_m, 4), "gbs": round(gbs, 1),
                                        "mfma_tflops_executed": round(mfma_flop / (kms_m * 1e-3) / 1e12, 1),
                                        "mfma_frac_of_bf16_peak": round(mfma_flop / (kms_m * 1e-3) / 1e12 /
                                                                        PEAK_F16_TFLOPS, 4)}},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode_moment"),
                         "algorithmic_bytes_per_call": alg,
                         "note": "single-read kernel; algorithmic bytes = one read of the K/V cache + q, P, out"},
            "two_pass": {"ms_per_call": round(dt2 * 1e3, 4), "tokens_per_s": round(wd.batch / dt2, 1),
                         "pass1": {"avg_ms": round(kms1, 4), "gbs": round(cache_bytes / (kms1 * 1e-3) / 1e9, 1),
                                   "traffic": t1},
                         "pass2": {"avg_ms": round(kms2, 4), "gbs": round(cache_bytes / (kms2 * 1e-3) / 1e9, 1),
                                   "traffic": t2},
                         "note": "two split-KV passes, each reading the cache once"}}
        log(f"decode {dt * 1e3:.3f} ms/call (single-read kernel {kms_m:.3f} ms, {gbs:.0f} GB/s); "
            f"two-pass {dt2 * 1e3:.3f} ms/call")

        # four new tokens per sequence (speculative decoding) against the same cache
        gq = torch.Generator(device=dev)
        gq.manual_seed(6)
        q4 = torch.randn((wd.batch, 4, wd.heads_q, wd.head_dim), generator=gq, device=dev).to(qd.dtype)
        for _ in range(2):
            plx.parallax_attn_decode(q4, kc, vc, Pd)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(Kd):
            plx.parallax_attn_decode(q4, kc, vc, Pd)
        torch.cuda.synchronize()
        dt4 = (time.perf_counter() - t0) / Kd
        result["decode"]["four_tokens"] = {"tokens_per_sequence": 4, "ms_per_call": round(dt4 * 1e3, 4),
                                           "tokens_per_s": round(4 * wd.batch / dt4, 1)}
        log(f"4-token decode {dt4 * 1e3:.3f} ms/call")
        del q4

        # the same keys in a shuffled pool of 256-key pages with a block table
        page = 256
        npb = wd.seqlen_k // page
        gperm = torch.Generator(device="cpu")
        gperm.manual_seed(5)
        perm = torch.randperm(wd.batch * npb, generator=gperm).to(dev)
        kp = torch.empty((wd.batch * npb, page, wd.heads_kv, wd.head_dim), dtype=kc.dtype, device=dev)
        kp[perm] = kc.reshape(wd.batch * npb, page, wd.heads_kv, wd.head_dim)
        del kc
        vp = torch.empty_like(kp)
        vp[perm] = vc.reshape(wd.batch * npb, page, wd.heads_kv, wd.head_dim)
        del vc
        table = perm.reshape(wd.batch, npb).to(torch.int32).contiguous()
        for _ in range(2):
            plx.parallax_attn_decode_paged(qd, kp, vp, table, Pd)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(Kd):
            plx.parallax_attn_decode_paged(qd, kp, vp, table, Pd)
        torch.cuda.synchronize()
        dtpg = (time.perf_counter() - t0) / Kd
        result["decode"]["paged"] = {"page_size": page, "ms_per_call": round(dtpg * 1e3, 4),
                                     "tokens_per_s": round(wd.batch / dtpg, 1),
                                     "gbs": round(alg / dtpg / 1e9, 1)}
        log(f"paged decode {dtpg * 1e3:.3f} ms/call")
        del kp, vp, table, perm

        if not args.no_sweep:
            # decode across batch sizes and context lengths (the pages' decode benchmark axes)
            sweep = []
            for Bs, Ls in ((1, 32768), (8, 32768), (64, 4096), (64, 16384), (256, 8192)):
                ws_ = W.scaled(wd, batch=Bs, seqlen_k=Ls)
                qs, ks, vs, Ps = W.make_inputs(ws_, device=dev)
                for _ in range(2):
                    plx.parallax_attn_decode(qs, ks, vs, Ps)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(5):
                    plx.parallax_attn_decode(qs, ks, vs, Ps)
                torch.cuda.synchronize()
                dts = (time.perf_counter() - t0) / 5
                by = 2 * Bs * Ls * ws_.heads_kv * ws_.head_dim * 2
                sweep.append({"batch": Bs, "context": Ls, "ms_per_call": round(dts * 1e3, 4),
                              "tokens_per_s": round(Bs / dts, 1), "gbs_one_read": round(by / dts / 1e9, 1)})
                log(f"decode sweep B={Bs} L={Ls}: {dts * 1e3:.3f} ms")
                del qs, ks, vs, Ps
            result["decode"]["sweep"] = sweep

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
