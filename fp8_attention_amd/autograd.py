"""``torch.autograd`` entry to the FP8 attention path.

``fp8_attention(q, k, v, causal, delta_mode)`` is a drop-in attention call whose
forward and backward run the library's kernels: the forward quantizes Q, K, V
into the block-scaled E4M3 operands each matmul contracts over and runs the
FP8 forward; the backward quantizes the incoming gradient dO to E5M2, computes
the row correction delta in the chosen mode and runs the FP8 backward
(Delta-Matching page, section 01 "Write down softmax backward" and "What
changes in FP8?"; section 03 for the matched correction).

Modes of delta (section 01 "Why can we reuse the forward output?" and section 03 of that page):
  * ``"matched"`` (default) -- sum_j P_ij dP^_ij from the backward's own FP8
    operands; the rows of dS then sum to zero up to FP32 rounding;
  * ``"do_matched"`` -- sum_k dO^_ik O_ik with the quantized dO;
  * ``"stale"`` -- sum_k dO_ik O_ik from the bf16 dO and the saved FP32 O.

Shapes: q [B, Hq, L, d_qk], k [B, Hkv, L, d_qk], v [B, Hkv, L, d_v] (Hq a
multiple of Hkv: grouped-query attention; dK and dV are summed over each
group), contiguous, bfloat16 or float32, on the GPU.  The output and the
gradients come back in the inputs' dtype.  dO enters the backward as bfloat16
(the stale mode is defined on the bf16 dO).  The context keeps the six FP8
operands (1 byte per element and layout plus the scales), the log-sum-exp and,
for the stale and dO-matched modes, which read it, the FP32 output.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import api

_QUANT = (("q_c", 0, "cols", "e4m3"), ("q_s", 0, "rows", "e4m3"), ("k_c", 1, "cols", "e4m3"),
          ("k_s", 1, "rows", "e4m3"), ("v_c", 2, "cols", "e4m3"), ("v_s", 2, "rows", "e4m3"))


def check_inputs(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, delta_mode: str) -> api.AttnShape:
    """Validate shapes, dtypes and layout; returns the problem shape (causal unset)."""
    if delta_mode not in api.MODES:
        raise ValueError(f"unknown delta mode {delta_mode!r}; expected one of {sorted(api.MODES)}")
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{n} must be [B, H, L, d], got shape {tuple(t.shape)}")
        if t.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError(f"{n} must be bfloat16 or float32, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    B, Hq, L, dqk = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if (Bk, Lk, dk) != (B, L, dqk) or tuple(v.shape[:3]) != (B, Hkv, L):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if Hkv == 0 or Hq % Hkv:
        raise ValueError(f"query heads ({Hq}) must be a multiple of KV heads ({Hkv})")
    return api.AttnShape(B, Hq, Hkv, L, dqk, v.shape[3], False)


class Fp8Attention(torch.autograd.Function):
    """Forward: FP8 attention.  Backward: delta in the chosen mode, then dQ, dK, dV."""

    @staticmethod
    def forward(ctx, q, k, v, causal: bool, delta_mode: str, softmax_scale: Optional[float]):
        s0 = check_inputs(q, k, v, delta_mode)
        shape = api.AttnShape(s0.batch, s0.heads_q, s0.heads_kv, s0.seqlen, s0.d_qk, s0.d_v, bool(causal),
                              softmax_scale)
        Lp = api.padded_len(shape.seqlen)
        src = (q, k, v)
        ops = {n: api.quantize(src[i], axis, fmt, Lp) for n, i, axis, fmt in _QUANT}
        o, lse = api.attn_fwd(shape, ops["q_c"], ops["k_c"], ops["v_s"])
        names = [n for n, *_ in _QUANT]
        ctx.names = names
        ctx.shape, ctx.mode, ctx.dtypes = shape, delta_mode, (q.dtype, k.dtype, v.dtype)
        # the FP32 output is read back only by the saved-output modes
        keep_o = o if delta_mode != "matched" else torch.empty(0, device=o.device)
        ctx.save_for_backward(keep_o, lse, *[t for n in names for t in ops[n]])
        return o if q.dtype == torch.float32 else o.to(q.dtype)

    @staticmethod
    def backward(ctx, grad_o):
        shape, mode = ctx.shape, ctx.mode
        o, lse, *flat = ctx.saved_tensors
        ops = {n: api.Fp8Operand(flat[2 * i], flat[2 * i + 1]) for i, n in enumerate(ctx.names)}
        do = grad_o.to(torch.bfloat16).contiguous()
        Lp = api.padded_len(shape.seqlen)
        ops["do_c"] = api.quantize(do, "cols", "e5m2", Lp)
        ops["do_s"] = api.quantize(do, "rows", "e5m2", Lp)
        if mode == "matched":
            delta = api.attn_delta(shape, mode, do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"], v_c=ops["v_c"],
                                   lse=lse)
        elif mode == "do_matched":
            delta = api.attn_delta(shape, mode, o=o, do_c=ops["do_c"])
        else:
            delta = api.attn_delta(shape, mode, o=o, do=do)
        # dK/dV through the head-split entry (a workspace only where the grid is small),
        # then dQ: the same kernels as the fused call otherwise
        g = api.attn_bwd_dkdv_ws(shape, ops, lse, delta)
        g.update(api.attn_bwd_dq(shape, ops, lse, delta))
        tq, tk, tv = ctx.dtypes
        return g["dq"].to(tq), g["dk"].to(tk), g["dv"].to(tv), None, None, None


def fp8_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                  delta_mode: str = "matched", softmax_scale: Optional[float] = None) -> torch.Tensor:
    """Block-scaled FP8 attention with a differentiable output; see the module docstring."""
    return Fp8Attention.apply(q, k, v, causal, delta_mode, softmax_scale)
