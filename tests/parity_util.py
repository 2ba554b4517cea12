"""Helpers shared by the GPU parity tests: run the oracle on a workload and compare.

The oracle always starts from the same bf16 bytes the GPU receives and from its
own quantization; nothing the GPU computes is fed into the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import attention as A
from fp8_attention_amd.workloads import Workload

REL_TOL = 2e-3          # max-abs error <= REL_TOL * RMS(oracle tensor) (+ cast-ambiguity radius)
ROWSUM_TOL = 1e-5       # |sum_j dS_ij| <= ROWSUM_TOL * sum_j |P_ij dP_ij| under Delta-Matching


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
    """Oracle forward + every requested delta mode + backward, with radii."""
    q, k, v, do = (to64(inputs[n]) for n in ("q", "k", "v", "do"))
    qops = A.quantize_operands(q, k, v, do)
    ops = A.decode_operands(qops, shp.seqlen)
    f = A.forward(ops, shp, rows=rows, radius=radius)
    out = {"qops": qops, "ops": ops, "fwd": f, "do": do}
    for mode in modes:
        d = A.delta(ops, shp, mode, o=f["o"], do=do, lse=f["lse"], rows=rows)
        out[mode] = {"delta": d, "bwd": A.backward(ops, shp, f["lse"], d, rows=rows, radius=radius)}
    return out


def compare(name: str, gpu, ref: np.ndarray, radius=None, rel: float = REL_TOL, mask=None) -> dict:
    """Assert |gpu - ref| <= rel * RMS(ref) + radius elementwise over finite ref entries."""
    g = to64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    ok = np.isfinite(ref)
    if mask is not None:
        ok &= mask
    assert ok.any(), f"{name}: nothing to compare"
    rms = float(np.sqrt(np.mean(ref[ok] ** 2)))
    err = np.abs(g - ref)
    base = rel * rms
    tol = base + (0.0 if radius is None else np.where(np.isfinite(radius), radius, 0.0))
    bad = ok & ~(err <= tol)
    stats = {"name": name, "rms": rms, "max_err_over_rms": float(err[ok].max() / max(rms, 1e-300)),
             "n": int(ok.sum()), "n_used_radius": int((ok & (err > base)).sum()), "n_bad": int(bad.sum())}
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(i) for i in ix), float(g[tuple(ix)]), float(ref[tuple(ix)]),
                   float(tol if np.isscalar(tol) else tol[tuple(ix)])) for ix in idx]
        raise AssertionError(f"{name}: {stats} first bad (index, gpu, oracle, tol): {detail}")
    return stats


def delta_tolerance(shp: A.Shape, ops: dict, lse, mode: str, o=None, do=None) -> np.ndarray:
    """Per-row bound of FP32 rounding in delta: TAU * sum of |terms| of its defining sum."""
    if mode == "matched":
        G = shp.group
        tol = np.zeros((shp.batch, shp.heads_q, shp.seqlen))
        for b in range(shp.batch):
            for h in range(shp.heads_q):
                P = A.probs_rows(ops["q_c"][b, h], ops["k_c"][b, h // G], lse[b, h], shp.sigma, shp.causal, 0,
                                 shp.seqlen)
                dP = ops["do_c"][b, h] @ ops["v_c"][b, h // G].T
                tol[b, h] = A.TAU * np.abs(P * dP).sum(axis=1)
        return tol
    x = do if mode == "stale" else ops["do_c"]
    return A.TAU * np.einsum("...k,...k->...", np.abs(x), np.abs(o))
