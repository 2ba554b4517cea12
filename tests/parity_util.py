"""Helpers shared by the GPU parity tests: run the oracle on a workload and compare.

The oracle always starts from the same bf16 bytes the GPU receives and from its
own quantization; nothing the GPU computes is fed into the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import attention as A
from fp8_attention_amd.workloads import Workload

REL_TOL = 2e-3          # max-abs error <= REL_TOL * RMS(oracle tensor) (+ allowance)
# Norm-wise bar on the deviation left once the oracle's cast-ambiguity radius is
# taken off each element.  The FP8 matrix instruction's own accumulation error
# and the cast flips it triggers are both legitimate; the flips are rare but one
# flip in a short, peaked row (the first rows under the causal mask) moves that
# row by several percent, enough to dominate the raw norm of a small test problem
# (1e-4 .. 1.5e-2 measured).  What remains after the radius is the accumulation
# error proper: at most 1.8e-5 of the norm on every test (2.7e-6 at full sizes).
# 1e-3 leaves room for the final product's accumulation error under strong
# cancellation (up to 2^-12.6 of sum |a b| per element) and is still a bar that a
# systematic error (a wrong scale, index or mask, which no flip explains) exceeds.
NORM_TOL = 1e-3
ROWSUM_TOL = 1e-5       # |sum_j dS_ij| <= ROWSUM_TOL * sum_j |P_ij dP_ij| under Delta-Matching

# Every comparison's statistics, printed in the session summary (tests/conftest.py),
# labelled with the running test (set by an autouse fixture there).
STATS: list = []
CURRENT_TEST = ""


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_shape(w: Workload, sigma: float, batch=None, hq=None, hkv=None) -> A.Shape:
    return A.Shape(batch or w.batch, hq or w.heads_q, hkv or w.heads_kv, w.seqlen, w.d_qk, w.d_v,
                   bool(w.causal), sigma)


def select_group(inputs: dict, w: Workload, b: int, g: int) -> dict:
    """Slice the bf16 inputs down to batch b and KV group g (its G query heads)."""
    G = w.group
    return {"q": inputs["q"][b:b + 1, g * G:(g + 1) * G], "k": inputs["k"][b:b + 1, g:g + 1],
            "v": inputs["v"][b:b + 1, g:g + 1], "do": inputs["do"][b:b + 1, g * G:(g + 1) * G]}


def run_oracle(inputs: dict, shp: A.Shape, modes=("matched",), rows=None, radius=True) -> dict:
    """Oracle forward + every requested delta mode + backward, with radii and bounds.

    The backward is evaluated with the oracle's own LSE and delta (float32
    rounding only), which is what the kernel-isolated tests feed the GPU.
    """
    q, k, v, do = (to64(inputs[n]) for n in ("q", "k", "v", "do"))
    qops = A.quantize_operands(q, k, v, do)
    ops = A.decode_operands(qops, shp.seqlen)
    f = A.forward(ops, shp, rows=rows, radius=radius)
    out = {"qops": qops, "ops": ops, "fwd": f, "do": do}
    for mode in modes:
        d = A.delta(ops, shp, mode, o=f["o"], do=do, lse=f["lse"], rows=rows)
        out[mode] = {"delta": d, "bwd": A.backward(ops, shp, f["lse"], d, rows=rows, radius=radius)}
    return out


def compare(name: str, gpu, ref: np.ndarray, allow=None, rel: float = REL_TOL, mask=None,
            norm_rel=None, flip=None, case: str = "") -> dict:
    """Assert |gpu - ref| <= rel * RMS(ref) + allow elementwise over finite ref entries.

    ``allow`` is the oracle's bound of how far a correct kernel result may sit
    from the exact value (ambiguous-cast radius plus the matrix cores'
    accumulation error).  With ``norm_rel`` also assert the norm-wise bar on the
    part of the deviation that no ambiguous cast explains:
    ||max(|gpu - ref| - flip, 0)||_2 <= norm_rel * ||ref||_2, where ``flip`` is the
    oracle's cast-ambiguity radius (a cast whose exact input lies within the
    kernel's error of a rounding boundary has two correct results; one such flip
    in a short, peaked row moves that row by several percent).

    The returned statistics split the elements beyond ``rel * RMS`` into those
    the flip radius explains, those the rest of the allowance (the matrix cores'
    accumulation bound) explains, and the unexplained ones (which fail).
    """
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    ok = np.isfinite(ref)
    if mask is not None:
        ok &= mask
    assert ok.any(), f"{name}: nothing to compare"
    rms = float(np.sqrt(np.mean(ref[ok] ** 2)))
    err = np.abs(g - ref)
    base = rel * rms
    tol = base + (0.0 if allow is None else np.where(np.isfinite(allow), allow, 0.0))
    bad = ok & ~(err <= tol)
    refn = max(np.sqrt(np.sum(ref[ok] ** 2)), 1e-300)
    nrel = float(np.sqrt(np.sum(err[ok] ** 2)) / refn)
    unexp = err if flip is None else np.maximum(err - np.where(np.isfinite(flip), flip, 0.0), 0.0)
    nrel_u = float(np.sqrt(np.sum(unexp[ok] ** 2)) / refn)
    fl = 0.0 if flip is None else np.where(np.isfinite(flip), flip, 0.0)
    beyond = ok & (err > base)
    by_flip = beyond & (err <= base + fl)
    stats = {"case": case or CURRENT_TEST, "name": name, "rms": rms, "max_err_over_rms": float(err[ok].max() / max(rms, 1e-300)),
             "norm_rel_err": nrel, "norm_rel_unexplained": nrel_u, "n": int(ok.sum()),
             "n_beyond_rel_rms": int(beyond.sum()), "n_flip_explained": int(by_flip.sum()),
             "n_accumulation_explained": int((beyond & ~by_flip & (err <= tol)).sum()), "n_bad": int(bad.sum())}
    STATS.append(stats)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(i) for i in ix), float(g[tuple(ix)]), float(ref[tuple(ix)]),
                   float(tol if np.isscalar(tol) else tol[tuple(ix)])) for ix in idx]
        raise AssertionError(f"{name}: {stats} first bad (index, gpu, oracle, tol): {detail}")
    if norm_rel is not None:
        assert nrel_u <= norm_rel, f"{name}: norm-wise relative error {nrel_u:.3e} > {norm_rel:.1e} ({stats})"
    return stats


def oracle_head_chain(q, k, v, do, shp: A.Shape, rows) -> dict:
    """Oracle chain (quantize, forward, matched delta with its bound, backward, with
    radii) for one query head given as float64 arrays [1, 1, L, d]; for the
    full-size tests, which run one head per worker process."""
    qops = A.quantize_operands(q, k, v, do)
    ops = A.decode_operands(qops, shp.seqlen)
    f = A.forward(ops, shp, rows=rows, radius=True)
    derr = A.delta_bound(ops, shp, "matched", lse=f["lse"], lse_err=f["b_lse"], rows=rows)
    d = A.delta(ops, shp, "matched", lse=f["lse"], rows=rows)
    r = A.backward(ops, shp, f["lse"], d, rows=rows, radius=True, delta_err=derr, lse_err=f["b_lse"])
    return {"qops": qops, "fwd": f, "delta": d, "derr": derr, "bwd": r}
