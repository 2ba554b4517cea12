"""Block-scaled FP8 attention forward, row correction and backward of the CPU oracle.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module.

All arithmetic is FP64 (numpy).  Matmuls are plain ``@`` products; nothing is
blocked, fused or reordered beyond processing query rows in independent ranges
to bound memory.  Sources ("Delta-Matching for reliable FP8 attention
training", the authors' project page; the display equations were lost in the
text copy, so each step cites the prose that defines it):

* Section 01, "Write down softmax backward": S = sigma * Q K^T with
  sigma = 1/sqrt(d), P = row softmax of S, O = P V; backward dV = P^T dO,
  dP = dO V^T, dS_ij = P_ij (dP_ij - delta_i) with delta_i = sum_j P_ij dP_ij,
  dQ = sigma dS K, dK = sigma dS^T Q.
* Section 01, "Why can we reuse the forward output?": the saved-output
  shortcut delta_i = sum_k dO_ik O_ik.
* Section 01, "What changes in FP8?": hatted operands are decoded FP8 values
  with their block scales; P is the FP32 softmax before probability
  quantization; O = P_hat V_hat and dP_hat = dO_hat V_hat^T with FP32
  accumulation; the stale correction uses dO before its FP8 cast.
* Section 03, "Does matching the backward operands fix it?": Delta-Matching
  takes delta_i = sum_j P_ij dP_hat_ij with P in FP32 and dP_hat the FP32
  product of the FP8 backward operands; all seven matmuls may use FP8 while
  softmax and reductions stay in higher precision; the dO-only variant
  replaces dO by dO_hat in the saved-output shortcut.

Readings where the page leaves a step open:

* FP8 formats: E4M3 for Q, K, V and P; E5M2 for dO and dS.  One power-of-two
  scale per 32 consecutive elements along each matmul's contraction axis.
* Which probabilities the forward quantizes: the unnormalised
  P'_ij = exp(S_ij - mu_i) where mu_i is the exact running row maximum over the
  keys seen so far, updated once per chunk of 128 consecutive keys; P' is cast
  in 32-key blocks, the normaliser l_i is summed from the *unquantized* P', and
  O is divided by l_i after the product.  LSE_i = m_i + ln l_i (natural log).
  The backward probabilities are P_ij = exp(S_ij - LSE_i).
* Causal masking keeps keys j <= i (queries and keys share one length L).
* GQA: query head h uses KV head h // (Hq / Hkv); dK and dV are summed over
  the query heads of a group.
* sigma multiplies the FP32 scores and the dQ/dK products; it is never folded
  into an operand before a cast.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import fp8

CHUNK = 128
BLOCK = fp8.BLOCK
# Error budget of a kernel's arithmetic, used only to decide which in-kernel
# casts are ambiguous and how far a correct kernel result may sit from the
# exact one:
#  TAU    relative rounding of the FP32 steps (exp2, scaling, sums): 128 ulps;
#  GAMMA  error of one FP8 matrix-core product, relative to sum_k |a_k b_k| of
#         that output.  The pages state FP32 accumulation; the gfx950 scaled FP8
#         instructions sum the products of each instruction with a narrower
#         adder.  Measured on the GPU against FP64 dot products
#         (tests/test_gpu_mfma_accumulation.py), for both instruction shapes the
#         kernels use and contraction lengths 64 to 2048: up to 2^-11.8 of
#         sum |a b| on softmax-shaped probability operands and 2^-11.4 on
#         same-sign codes spanning the whole format, independent of the number
#         of chained instructions, and an accumulator input (the dP products
#         that start from -delta) is carried to within a few FP32 ulps of the
#         result, which TAU covers.  2^-11 is the smallest power of two above
#         every measured case.
TAU = 2.0 ** -17
GAMMA = 2.0 ** -11

MODES = ("stale", "do_matched", "matched")


@dataclasses.dataclass(frozen=True)
class Shape:
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    d_qk: int
    d_v: int
    causal: bool
    sigma: float

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv


def _roundup(x: int, m: int) -> int:
    return (x + m - 1) // m * m


# ---------------------------------------------------------------------------
# Operand quantization (what the library's quantize call must reproduce bit for bit)
# ---------------------------------------------------------------------------

def quantize_channels(x: np.ndarray, fmt):
    """Blocks of 32 along the last (channel) axis: codes [..., L, d], scales [..., L, d/32]."""
    codes, scales, _ = fp8.quantize_lastaxis(np.asarray(x, dtype=np.float64), fmt)
    return codes, scales


def quantize_sequence(x: np.ndarray, fmt):
    """Blocks of 32 along the sequence axis, stored transposed so blocks are contiguous.

    x [..., L, d] -> codes [..., d, L32], scales [..., d, L32/32] with L32 = roundup(L, 32);
    the positions past L hold zeros (they do not change any block amax).
    """
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[-2]
    L32 = _roundup(L, BLOCK)
    xt = np.zeros(x.shape[:-2] + (x.shape[-1], L32))
    xt[..., :L] = np.swapaxes(x, -1, -2)
    codes, scales, _ = fp8.quantize_lastaxis(xt, fmt)
    return codes, scales


def dequantize_channels(codes, scales, fmt) -> np.ndarray:
    return fp8.dequantize_lastaxis(codes, scales, fmt)


def dequantize_sequence(codes, scales, fmt, L: int) -> np.ndarray:
    xt = fp8.dequantize_lastaxis(codes, scales, fmt)
    return np.ascontiguousarray(np.swapaxes(xt[..., :L], -1, -2))


def quantize_operands(q, k, v, do):
    """All eight FP8 operands from the bf16 inputs (given as float arrays).

    Returns {name: (codes, scales)} for q_c, k_c, v_c, do_c (channel blocks) and
    q_s, k_s, v_s, do_s (sequence blocks, transposed).
    """
    out = {}
    for name, x, fmt in (("q", q, "e4m3"), ("k", k, "e4m3"), ("v", v, "e4m3"), ("do", do, "e5m2")):
        out[name + "_c"] = quantize_channels(x, fmt)
        out[name + "_s"] = quantize_sequence(x, fmt)
    return out


FORMAT_OF = {"q": "e4m3", "k": "e4m3", "v": "e4m3", "do": "e5m2"}


def decode_operands(qops: dict, L: int) -> dict:
    """FP64 values of the quantized operands, all in [B, H, L, d] orientation."""
    out = {}
    for key, (codes, scales) in qops.items():
        base, axis = key.rsplit("_", 1)
        fmt = FORMAT_OF[base]
        if axis == "c":
            out[key] = dequantize_channels(codes, scales, fmt)
        else:
            out[key] = dequantize_sequence(codes, scales, fmt, L)
    return out


# ---------------------------------------------------------------------------
# Per-head, per-row-range kernels of the definition
# ---------------------------------------------------------------------------

def _scores(Qr, K, sigma, r0, causal, Lk):
    """S = sigma Q K^T for query rows r0.. (FP64), -inf where masked.  Key axis padded to Lk."""
    n = Qr.shape[0]
    L = K.shape[0]
    S = np.full((n, Lk), -np.inf)
    S[:, :L] = sigma * (Qr @ K.T)
    if causal:
        i = np.arange(r0, r0 + n)[:, None]
        j = np.arange(Lk)[None, :]
        S[j > i] = -np.inf
    return S


def _abs_scores(Qr, K, sigma, Lk):
    n = Qr.shape[0]
    A = np.zeros((n, Lk))
    A[:, :K.shape[0]] = abs(sigma) * (np.abs(Qr) @ np.abs(K).T)
    return A


def forward_rows(Q, K, V, sigma, causal, r0, r1, cast=True, radius=False):
    """Forward for query rows [r0, r1) of one head.

    Q [L, dqk], K [L, dqk], V [L, dv] are the decoded operands the two forward
    matmuls use (Q_hat<c>, K_hat<c>, V_hat<s>).  Returns O and LSE; with
    ``radius`` also
      r_o   first-order bound of how far O may move because probability casts
            whose exact input lies within the kernel's error budget of a
            rounding or scale boundary can go either way (both are correct);
      b_o   bound of the kernel's own accumulation error in O (GAMMA on the
            P V product, and the score error carried through mu and l);
      b_lse bound of the kernel's LSE error.
    """
    L = K.shape[0]
    Lc = _roundup(L, CHUNK)
    S = _scores(Q[r0:r1], K, sigma, r0, causal, Lc)
    n = S.shape[0]
    nc = Lc // CHUNK
    cmax = S.reshape(n, nc, CHUNK).max(axis=2)
    mu = np.maximum.accumulate(cmax, axis=1)                  # running max per chunk
    mu_full = np.repeat(mu, CHUNK, axis=1)
    finite = np.isfinite(mu_full)
    with np.errstate(invalid="ignore"):
        Pp = np.where(finite, np.exp(S - np.where(finite, mu_full, 0.0)), 0.0)
    m = mu[:, -1]
    l = np.exp(S - m[:, None]).sum(axis=1)
    lse = m + np.log(l)
    err = None
    if radius:
        live = np.isfinite(S)
        eS = np.where(live, GAMMA * _abs_scores(Q[r0:r1], K, sigma, Lc) + TAU * (np.abs(np.where(live, S, 0)) + 1),
                      0.0)
        E = eS.max(axis=1)                                     # the row maximum's own error bounds mu's
        err = Pp * (eS + E[:, None] + TAU * (np.abs(np.where(live, S, 0) - np.where(finite, mu_full, 0)) + 1))
    if cast:
        Ph, dPh, ne, nb = fp8.cast_lastaxis(Pp, fp8.E4M3, err)
    else:
        Ph, dPh, ne, nb = Pp, (np.zeros_like(Pp) if radius else None), 0, 0
    w = np.where(finite, np.exp(np.where(finite, mu_full, 0.0) - m[:, None]), 0.0) / l[:, None]
    O = (Ph * w)[:, :L] @ V
    out = {"o": O, "lse": lse, "n_flag": ne, "n_block_flag": nb}
    if radius:
        out["r_o"] = (dPh * w)[:, :L] @ np.abs(V)
        out["b_o"] = GAMMA * (np.abs(Ph * w)[:, :L] @ np.abs(V)) + 2 * E[:, None] * np.abs(O)
        out["b_lse"] = 2 * E + TAU * (np.abs(lse) + 1)
    return out


def probs_rows(Q, K, lse, sigma, causal, r0, r1):
    """Backward FP32-role probabilities P_ij = exp(S_ij - LSE_i) for rows [r0, r1)."""
    L = K.shape[0]
    S = _scores(Q[r0:r1], K, sigma, r0, causal, L)
    return np.exp(S - lse[:, None])


def delta_rows(mode, r0, r1, *, O=None, dO=None, dOc=None, Q=None, K=None, Vc=None,
               lse=None, sigma=None, causal=None):
    """Row correction delta for rows [r0, r1) of one head."""
    if mode == "stale":
        return np.einsum("ik,ik->i", dO[r0:r1], O)
    if mode == "do_matched":
        return np.einsum("ik,ik->i", dOc[r0:r1], O)
    if mode == "matched":
        P = probs_rows(Q, K, lse, sigma, causal, r0, r1)
        dP = dOc[r0:r1] @ Vc.T
        return (P * dP).sum(axis=1)
    raise ValueError(f"unknown delta mode {mode!r}")


def _pad_rows(x, n32):
    if x.shape[0] == n32:
        return x
    out = np.zeros((n32,) + x.shape[1:])
    out[:x.shape[0]] = x
    return out


def backward_rows(ops_h, lse, delta, sigma, causal, r0, r1, cast=True, radius=False,
                  delta_err=None, lse_err=None, keep_ds=False):
    """Backward for query rows [r0, r1) of one head (r0 % 32 == 0; r1 % 32 == 0 or r1 == L).

    ``ops_h`` holds the decoded operands of this head: q_c, k_c, v_c, do_c,
    q_s, k_s, do_s as [L, d].  Returns dQ for the rows, and the partial dK, dV
    contributed by these rows (sum them over row ranges and the heads of a group),
    and per row: the sum of dS before its casts ("rowsum"), of |P dP_hat|
    ("rowabs") and of dS^<k> after its E5M2 cast along keys ("rowsum_cast": the
    residual the cast adds once Delta-Matching has removed the pre-cast one,
    project page section 03).  With ``radius`` also the flip radii r_* and
    accumulation bounds b_* of dq, dk, dv, b_rowsum, and r_/b_rowsum_cast.
    ``delta_err`` / ``lse_err`` bound how far the delta and LSE the kernel is
    given may sit from the exact ones (default: float32 rounding).  ``keep_ds``
    also returns the pre-cast dS of the rows ("ds").
    """
    Q, K, Vc = ops_h["q_c"], ops_h["k_c"], ops_h["v_c"]
    dOc, Qs, Ks, dOs = ops_h["do_c"], ops_h["q_s"], ops_h["k_s"], ops_h["do_s"]
    L = K.shape[0]
    L32 = _roundup(L, BLOCK)
    n = r1 - r0
    n32 = _roundup(n, BLOCK)
    S = _scores(Q[r0:r1], K, sigma, r0, causal, L32)
    P = np.exp(S - lse[:, None])                                   # FP32-role probabilities
    dP = np.zeros((n, L32))
    dP[:, :L] = dOc[r0:r1] @ Vc.T                                  # dP_hat
    dS = P * (dP - delta[:, None])
    rowsum = dS.sum(axis=1)
    rowabs = np.abs(P * dP).sum(axis=1)
    errP = errS = None
    if radius:
        live = np.isfinite(S)
        Sl = np.where(live, S, 0.0)
        eS = np.where(live, GAMMA * _abs_scores(Q[r0:r1], K, sigma, L32) + TAU * (np.abs(Sl) + 1), 0.0)
        B = np.zeros((n, L32))
        B[:, :L] = np.abs(dOc[r0:r1]) @ np.abs(Vc).T
        edP = GAMMA * B + TAU * np.abs(dP)
        eL = TAU * (np.abs(lse) + 1) if lse_err is None else np.asarray(lse_err) + TAU * (np.abs(lse) + 1)
        eD = TAU * (np.abs(delta) + rowabs) if delta_err is None else np.asarray(delta_err) + TAU * rowabs
        eP = eS + eL[:, None] + TAU * (np.abs(Sl - lse[:, None]) + 1)   # relative error of P
        errP = P * eP
        errS = P * (edP + eD[:, None] + TAU * (np.abs(dP) + np.abs(delta)[:, None])) + np.abs(dS) * eP
        b_rowsum = (P * edP).sum(axis=1) + (np.abs(dS) * eP).sum(axis=1) + eD * P.sum(axis=1) + TAU * rowabs
    if cast:
        Pq, dPq, n1, b1 = fp8.cast_axis(_pad_rows(P, n32), fp8.E4M3, 0,
                                        None if errP is None else _pad_rows(errP, n32))
        dSk, ddSk, n2, b2 = fp8.cast_lastaxis(dS, fp8.E5M2, errS)
        dSq, ddSq, n3, b3 = fp8.cast_axis(_pad_rows(dS, n32), fp8.E5M2, 0,
                                          None if errS is None else _pad_rows(errS, n32))
        Pq, dSq = Pq[:n], dSq[:n]
        if radius:
            dPq, ddSq = dPq[:n], ddSq[:n]
        flags = (n1 + n2 + n3, b1 + b2 + b3)
    else:
        Pq, dSk, dSq = P, dS, dS
        if radius:
            dPq = ddSk = ddSq = np.zeros_like(P)
        flags = (0, 0)
    out = {
        "dq": sigma * (dSk[:, :L] @ Ks),
        "dk": sigma * (dSq[:, :L].T @ Qs[r0:r1]),
        "dv": Pq[:, :L].T @ dOs[r0:r1],
        "rowsum": rowsum,
        "rowabs": rowabs,
        "rowsum_cast": dSk[:, :L].sum(axis=1),
        "n_flag": flags[0],
        "n_block_flag": flags[1],
    }
    if radius:
        aK, aQ, aO = np.abs(Ks), np.abs(Qs[r0:r1]), np.abs(dOs[r0:r1])
        out["r_dq"] = abs(sigma) * (ddSk[:, :L] @ aK)
        out["r_dk"] = abs(sigma) * (ddSq[:, :L].T @ aQ)
        out["r_dv"] = dPq[:, :L].T @ aO
        out["b_dq"] = GAMMA * abs(sigma) * (np.abs(dSk[:, :L]) @ aK)
        out["b_dk"] = GAMMA * abs(sigma) * (np.abs(dSq[:, :L]).T @ aQ)
        out["b_dv"] = GAMMA * (np.abs(Pq[:, :L]).T @ aO)
        out["b_rowsum"] = b_rowsum
        out["r_rowsum_cast"] = ddSk[:, :L].sum(axis=1)
        out["b_rowsum_cast"] = TAU * np.abs(dSk[:, :L]).sum(axis=1)
    if keep_ds:
        out["ds"] = dS[:, :L]
    return out


def delta_bound_rows(mode, r0, r1, *, O=None, dO=None, dOc=None, Q=None, K=None, Vc=None, lse=None,
                     sigma=None, causal=None, o_err=None, lse_err=None):
    """Bound of |delta_kernel - delta_exact| for rows [r0, r1) of one head.

    Saved-output modes: FP32 rounding of the dot product plus the deviation
    ``o_err`` of the O the kernel reads.  Matched mode: the kernel's errors in
    S (through P) and in dP_hat (GAMMA-bounded products), the error ``lse_err``
    of the LSE it reads, and FP32 rounding of the sum.
    """
    if mode in ("stale", "do_matched"):
        x = dO[r0:r1] if mode == "stale" else dOc[r0:r1]
        b = TAU * np.einsum("ik,ik->i", np.abs(x), np.abs(O))
        if o_err is not None:
            b = b + np.einsum("ik,ik->i", np.abs(x), o_err)
        return b
    L = K.shape[0]
    S = _scores(Q[r0:r1], K, sigma, r0, causal, L)
    live = np.isfinite(S)
    Sl = np.where(live, S, 0.0)
    P = np.exp(S - lse[:, None])
    dP = dOc[r0:r1] @ Vc.T
    eS = np.where(live, GAMMA * _abs_scores(Q[r0:r1], K, sigma, L) + TAU * (np.abs(Sl) + 1), 0.0)
    eL = TAU * (np.abs(lse) + 1) if lse_err is None else np.asarray(lse_err) + TAU * (np.abs(lse) + 1)
    edP = GAMMA * (np.abs(dOc[r0:r1]) @ np.abs(Vc).T) + TAU * np.abs(dP)
    pdp = np.abs(P * dP)
    return (P * edP).sum(axis=1) + (pdp * (eS + eL[:, None])).sum(axis=1) + TAU * pdp.sum(axis=1)


# ---------------------------------------------------------------------------
# Whole-tensor entry points (mirror the library's calls)
# ---------------------------------------------------------------------------

def _ranges(L, rows, step):
    if rows is None:
        rows = [(0, L)]
    out = []
    for a, b in rows:
        if a % BLOCK or (b % BLOCK and b != L) or not (0 <= a < b <= L):
            raise ValueError(f"row range {(a, b)} must be 32-aligned within [0, {L}]")
        for s in range(a, b, step):
            out.append((s, min(b, s + step)))
    return out


def _row_mask(L, rows):
    m = np.zeros(L, dtype=bool)
    for a, b in (rows or [(0, L)]):
        m[a:b] = True
    return m


def _step_for(L):
    # bound each [rows x keys] FP64 temporary to about 64 MB
    return max(BLOCK, min(L, (8 * 1024 * 1024) // max(L, 1) // BLOCK * BLOCK))


def forward(ops: dict, shp: Shape, rows=None, cast=True, radius=False) -> dict:
    """O [B,Hq,L,dv], LSE [B,Hq,L] (+ r_o, b_o, b_lse with ``radius``); rows outside ``rows`` are NaN."""
    B, Hq, L = shp.batch, shp.heads_q, shp.seqlen
    G = shp.group
    O = np.full((B, Hq, L, shp.d_v), np.nan)
    LSE = np.full((B, Hq, L), np.nan)
    extra = {k: np.full_like(O, np.nan) for k in ("r_o", "b_o")} if radius else {}
    if radius:
        extra["b_lse"] = np.full_like(LSE, np.nan)
    nflag = nblock = 0
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r0, r1 in _ranges(L, rows, _step_for(L)):
                f = forward_rows(ops["q_c"][b, h], ops["k_c"][b, g], ops["v_s"][b, g], shp.sigma,
                                 shp.causal, r0, r1, cast=cast, radius=radius)
                O[b, h, r0:r1] = f["o"]
                LSE[b, h, r0:r1] = f["lse"]
                nflag += f["n_flag"]
                nblock += f["n_block_flag"]
                for k in extra:
                    extra[k][b, h, r0:r1] = f[k]
    return {"o": O, "lse": LSE, "n_flag": nflag, "n_block_flag": nblock, **extra}


def _delta_args(ops, shp, mode, b, h, r0, r1, o, do, lse):
    g = h // shp.group
    if mode == "matched":
        return dict(dOc=ops["do_c"][b, h], Q=ops["q_c"][b, h], K=ops["k_c"][b, g], Vc=ops["v_c"][b, g],
                    lse=lse[b, h, r0:r1], sigma=shp.sigma, causal=shp.causal)
    return dict(O=o[b, h, r0:r1], dO=None if do is None else do[b, h], dOc=ops["do_c"][b, h])


def delta(ops: dict, shp: Shape, mode: str, *, o=None, do=None, lse=None, rows=None) -> np.ndarray:
    """delta [B,Hq,L] in one of the three modes; rows outside ``rows`` are NaN.

    stale      : rowsum(dO * O) with dO before its FP8 cast (``do``, [B,Hq,L,dv]);
    do_matched : rowsum(dO_hat<c> * O);
    matched    : rowsum(P * dP_hat), P = exp(S - LSE), dP_hat = dO_hat<c> V_hat<c>^T.
    """
    if mode not in MODES:
        raise ValueError(f"unknown delta mode {mode!r}")
    B, Hq, L = shp.batch, shp.heads_q, shp.seqlen
    D = np.full((B, Hq, L), np.nan)
    for b in range(B):
        for h in range(Hq):
            for r0, r1 in _ranges(L, rows, _step_for(L)):
                D[b, h, r0:r1] = delta_rows(mode, r0, r1, **_delta_args(ops, shp, mode, b, h, r0, r1, o, do, lse))
    return D


def delta_bound(ops: dict, shp: Shape, mode: str, *, o=None, do=None, lse=None, rows=None, o_err=None,
                lse_err=None) -> np.ndarray:
    """Per-row bound of |delta_kernel - delta_exact| (see delta_bound_rows)."""
    B, Hq, L = shp.batch, shp.heads_q, shp.seqlen
    D = np.full((B, Hq, L), np.nan)
    for b in range(B):
        for h in range(Hq):
            for r0, r1 in _ranges(L, rows, _step_for(L)):
                kw = _delta_args(ops, shp, mode, b, h, r0, r1, o, do, lse)
                if mode == "matched":
                    kw["lse_err"] = None if lse_err is None else lse_err[b, h, r0:r1]
                else:
                    kw["o_err"] = None if o_err is None else o_err[b, h, r0:r1]
                D[b, h, r0:r1] = delta_bound_rows(mode, r0, r1, **kw)
    return D


def backward(ops: dict, shp: Shape, lse, delt, rows=None, cast=True, radius=False,
             delta_err=None, lse_err=None) -> dict:
    """dQ [B,Hq,L,dqk], dK [B,Hkv,L,dqk], dV [B,Hkv,L,dv] and the row-sum probes.

    With ``rows`` only those query rows contribute: dQ and the probes are NaN
    elsewhere, and dK/dV are exact only for keys whose every contributing query
    lies inside ``rows`` (with causal masking: keys j >= the first row of the
    last contiguous range that reaches L).  With ``radius`` also r_* (flip
    radii), b_* (accumulation bounds) and b_rowsum; ``delta_err`` / ``lse_err``
    [B,Hq,L] bound the deviation of the delta / LSE the kernel is given.
    """
    B, Hq, Hkv, L = shp.batch, shp.heads_q, shp.heads_kv, shp.seqlen
    G = shp.group
    dQ = np.full((B, Hq, L, shp.d_qk), np.nan)
    dK = np.zeros((B, Hkv, L, shp.d_qk))
    dV = np.zeros((B, Hkv, L, shp.d_v))
    rs = np.full((B, Hq, L), np.nan)
    ra = np.full((B, Hq, L), np.nan)
    rc = np.full((B, Hq, L), np.nan)
    ext = {}
    if radius:
        ext = {"r_dq": np.full_like(dQ, np.nan), "b_dq": np.full_like(dQ, np.nan),
               "r_dk": np.zeros_like(dK), "b_dk": np.zeros_like(dK),
               "r_dv": np.zeros_like(dV), "b_dv": np.zeros_like(dV), "b_rowsum": np.full_like(rs, np.nan),
               "r_rowsum_cast": np.full_like(rs, np.nan), "b_rowsum_cast": np.full_like(rs, np.nan)}
    nflag = nblock = 0
    for b in range(B):
        for h in range(Hq):
            g = h // G
            oh = {"q_c": ops["q_c"][b, h], "k_c": ops["k_c"][b, g], "v_c": ops["v_c"][b, g],
                  "do_c": ops["do_c"][b, h], "q_s": ops["q_s"][b, h], "k_s": ops["k_s"][b, g],
                  "do_s": ops["do_s"][b, h]}
            for r0, r1 in _ranges(L, rows, _step_for(L)):
                de = None if delta_err is None else delta_err[b, h, r0:r1]
                le = None if lse_err is None else lse_err[b, h, r0:r1]
                r = backward_rows(oh, lse[b, h, r0:r1], delt[b, h, r0:r1], shp.sigma, shp.causal,
                                  r0, r1, cast=cast, radius=radius, delta_err=de, lse_err=le)
                dQ[b, h, r0:r1] = r["dq"]
                dK[b, g] += r["dk"]
                dV[b, g] += r["dv"]
                rs[b, h, r0:r1] = r["rowsum"]
                ra[b, h, r0:r1] = r["rowabs"]
                rc[b, h, r0:r1] = r["rowsum_cast"]
                nflag += r["n_flag"]
                nblock += r["n_block_flag"]
                if radius:
                    ext["r_dq"][b, h, r0:r1] = r["r_dq"]
                    ext["b_dq"][b, h, r0:r1] = r["b_dq"]
                    ext["b_rowsum"][b, h, r0:r1] = r["b_rowsum"]
                    ext["r_rowsum_cast"][b, h, r0:r1] = r["r_rowsum_cast"]
                    ext["b_rowsum_cast"][b, h, r0:r1] = r["b_rowsum_cast"]
                    for k in ("r_dk", "b_dk", "r_dv", "b_dv"):
                        ext[k][b, g] += r[k]
    return {"dq": dQ, "dk": dK, "dv": dV, "rowsum": rs, "rowabs": ra, "rowsum_cast": rc,
            "n_flag": nflag, "n_block_flag": nblock, **ext}
