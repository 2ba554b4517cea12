"""Benchmark of the block-scaled FP8 attention path on one MI355X.

One step = forward + Delta-Matching row correction + backward (the whole hot
path) over one batch of synthetic inputs already quantized and resident in
HBM.  Prints one JSON line: the 7-matmul FP8 attention TFLOP/s of the long-
context GQA workload (B=4, 32 query / 8 KV heads, L=8192, d=128, causal), the
roofline of the dominant kernel, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fp8_attention_amd import workloads as W  # noqa: E402

METRIC = "FP8 attn fwd+bwd TFLOP/s (7 matmuls) at L=8K d=128 causal; % FP8 MFMA peak"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 matrix throughput
PEAK_HBM_GBS = 8000.0


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _pairs(w) -> float:
    return w.seqlen * w.seqlen / (2.0 if w.causal else 1.0) * w.batch * w.heads_q


# Matmul FLOPs each kernel executes (its own recomputation of S and dP^ included):
#   forward  S, P'V            2 (d_qk + d_v) per pair
#   delta    S, dP^            2 (d_qk + d_v)
#   dK/dV    S, dP^, dV, dK    2 (2 d_qk + 2 d_v)
#   dQ       S, dP^, dQ        2 (2 d_qk + d_v)
def fwd_flops(w) -> float:
    return 2.0 * (w.d_qk + w.d_v) * _pairs(w)


def dkdv_flops(w) -> float:
    return 2.0 * (2 * w.d_qk + 2 * w.d_v) * _pairs(w)


def dq_flops(w) -> float:
    return 2.0 * (2 * w.d_qk + w.d_v) * _pairs(w)


def cpu_baseline(w, inputs, rows: int) -> dict:
    """The oracle (untuned) on one batch entry and KV group, for the last ``rows`` query rows."""
    from oracle import attention as A
    from tests.parity_util import select_group, to64
    sel = select_group(inputs, w, w.batch - 1, w.heads_kv - 1)
    L = w.seqlen
    shp = A.Shape(1, w.group, 1, L, w.d_qk, w.d_v, w.causal, 1.0 / np.sqrt(w.d_qk))
    t0 = time.perf_counter()
    q, k, v, do = (to64(sel[n]) for n in ("q", "k", "v", "do"))
    ops = A.decode_operands(A.quantize_operands(q, k, v, do), L)
    r = [(L - rows, L)]
    f = A.forward(ops, shp, rows=r)
    d = A.delta(ops, shp, "matched", lse=f["lse"], rows=r)
    A.backward(ops, shp, f["lse"], d, rows=r)
    dt = time.perf_counter() - t0
    i = np.arange(L - rows, L)
    pairs = float((i + 1).sum()) if w.causal else float(rows * L)
    flops = 2.0 * (4 * w.d_qk + 3 * w.d_v) * pairs * w.group
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": dt,
            "sample": f"one batch entry x one KV group ({w.group} query heads), last {rows} of {L} query rows "
                      f"(forward, matched delta, backward incl. FP8 operand quantization); 7-matmul FLOPs of "
                      f"that sample / wall time; numpy FP64"}


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter summary, or None when the
    summary is for another workload or the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    k = rec.get("kernels", {}).get(kernel)
    if rec.get("workload") != workload or k is None:
        return None
    h = hashlib.sha256()
    for f in k["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != k["sha256"]:
        return None
    return k["hbm_read_bytes"] + k["hbm_write_bytes"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_8k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", action="store_true", help="also time quantize and the saved-output delta modes")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB three times (for calibrating rocprofv3's "
                         "FETCH_SIZE / WRITE_SIZE against a known byte count) and exit")
    args = ap.parse_args()
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        c = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            c.copy_(a)
        torch.cuda.synchronize()
        _log(f"[bench] copied {n} bytes three times")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested); the path has no multi-GPU form.",
              file=sys.stderr)
        sys.exit(2)

    from fp8_attention_amd import api
    w = W.WORKLOADS[args.workload]
    _log(f"[bench] workload {w}")
    inputs = W.generate(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal)
    torch.cuda.synchronize()
    tq0 = time.perf_counter()
    ops = api.quantize_operands(dev["q"], dev["k"], dev["v"], dev["do"])
    torch.cuda.synchronize()
    _log(f"[bench] first quantize {1e3 * (time.perf_counter() - tq0):.2f} ms (includes first-launch costs)")

    B, Hq, L = w.batch, w.heads_q, w.seqlen
    o = torch.empty((B, Hq, L, w.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq = torch.empty((B, Hq, L, w.d_qk), dtype=torch.float32, device="cuda")
    dk = torch.empty((B, w.heads_kv, L, w.d_qk), dtype=torch.float32, device="cuda")
    dv = torch.empty((B, w.heads_kv, L, w.d_v), dtype=torch.float32, device="cuda")
    # dK/dV workspace for the head split of small grids (none at the long-context sizes)
    ws_bytes = api.dkdv_workspace_size(shape)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    _log(f"[bench] dK/dV head-split workspace {ws_bytes} bytes")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        api.attn_fwd(shape, ops["q_c"], ops["k_c"], ops["v_s"], o=o, lse=lse)
        if ev is not None:
            ev[1].record()
        api.attn_delta(shape, "matched", do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"], v_c=ops["v_c"],
                       lse=lse, out=delta)
        if ev is not None:
            ev[2].record()
        api.attn_bwd_dkdv_ws(shape, ops, lse, delta, workspace=ws, dk=dk, dv=dv)
        if ev is not None:
            ev[3].record()
        api.attn_bwd_dq(shape, ops, lse, delta, dq=dq)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly K steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1e3 * elapsed / args.steps
    k_fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    k_del = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    k_dkdv = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    k_dq = float(np.mean([e[3].elapsed_time(e[4]) for e in evs]))
    flops = w.matmul_flops()
    value = flops / (ms_step * 1e-3) / 1e12
    _log(f"[bench] ms/step {ms_step:.3f} (fwd {k_fwd:.3f}, matched delta {k_del:.3f}, dkdv {k_dkdv:.3f}, "
         f"dq {k_dq:.3f}) "
         f"-> {value:.1f} TFLOP/s = {100 * value / PEAK_FP8_TFLOPS:.1f}% of FP8 peak")
    kern = {"fwd": (k_fwd, fwd_flops(w)), "delta_matched": (k_del, fwd_flops(w)),
            "bwd_dkdv": (k_dkdv, dkdv_flops(w)), "bwd_dq": (k_dq, dq_flops(w))}
    dom = max(kern, key=lambda n: kern[n][0])
    ach = kern[dom][1] / (kern[dom][0] * 1e-3) / 1e12
    extra = {n: {"ms": t, "tflops_algorithmic": f / (t * 1e-3) / 1e12} for n, (t, f) in kern.items()}

    if args.extra:
        def timeit(fn, n=5):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n
        tq = timeit(lambda: api.quantize_operands(dev["q"], dev["k"], dev["v"], dev["do"]))
        nel = sum(t.numel() for t in dev.values())
        qbytes = nel * 2 * (2 + 2 * (1 + 4 / 32)) / 2     # per operand: 2 B in, 2 x 1.125 B out
        ts = timeit(lambda: api.attn_delta(shape, "stale", o=o, do=dev["do"], out=delta))
        td = timeit(lambda: api.attn_delta(shape, "do_matched", o=o, do_c=ops["do_c"], out=delta))
        rows = B * Hq * L
        extra["quantize_all8"] = {"ms": tq, "GBps_algorithmic": qbytes / (tq * 1e-3) / 1e9}
        extra["delta_stale"] = {"ms": ts, "GBps_algorithmic": rows * (w.d_v * 6 + 4) / (ts * 1e-3) / 1e9}
        extra["delta_do_matched"] = {"ms": td,
                                     "GBps_algorithmic": rows * (w.d_v * (4 + 1 + 4 / 32) + 4) / (td * 1e-3) / 1e9}
        _log(f"[bench] extra {json.dumps(extra)}")

    cpu = None
    if not args.no_cpu_baseline:
        _log(f"[bench] CPU oracle baseline on a sample ({args.cpu_rows} rows) ...")
        cpu = cpu_baseline(w, inputs, args.cpu_rows)
        _log(f"[bench] CPU oracle {cpu['seconds']:.1f} s -> {cpu['value']:.6f} TFLOP/s on {cpu['cores']} cores")

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8(e4m3/e5m2)->fp32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seqlen": w.seqlen, "d_qk": w.d_qk, "d_v": w.d_v, "causal": w.causal,
                   "delta_mode": "matched", "step": "fwd + matched delta + bwd on pre-quantized operands",
                   "pct_fp8_peak": 100 * value / PEAK_FP8_TFLOPS},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_FP8_TFLOPS, "traffic": measured_traffic(w.name, dom)},
        "kernels": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
