"""Python binding of libdm: argument marshalling only.

Every step of the attention path runs in the library's HIP kernels; this
module only allocates output tensors with PyTorch (device memory), passes raw
pointers and the current HIP stream through ctypes, and raises on a non-OK
status.  Names follow the C ABI in include/dm_attn.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import NamedTuple, Optional

import torch

from . import _lib
from ._lib import DmError  # noqa: F401  (raised by every call on a non-zero status)

MODES = {"stale": _lib.DM_DELTA_STALE, "do_matched": _lib.DM_DELTA_DO_MATCHED, "matched": _lib.DM_DELTA_MATCHED}
FORMATS = {"e4m3": _lib.DM_E4M3, "e5m2": _lib.DM_E5M2}
AXES = {"cols": _lib.DM_AXIS_COLS, "rows": _lib.DM_AXIS_ROWS}
# operand -> FP8 format: E4M3 forward operands, E5M2 gradients
OPERAND_FORMAT = {"q": "e4m3", "k": "e4m3", "v": "e4m3", "do": "e5m2"}


class Fp8Operand(NamedTuple):
    codes: torch.Tensor    # uint8
    scales: torch.Tensor   # float32 powers of two, one per 32 codes

    def c(self) -> _lib.Operand:
        return _lib.Operand(self.codes.data_ptr(), self.scales.data_ptr())


_NULL_OPERAND = _lib.Operand(None, None)


@dataclasses.dataclass(frozen=True)
class AttnShape:
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    d_qk: int
    d_v: int
    causal: bool
    softmax_scale: Optional[float] = None

    @property
    def sigma(self) -> float:
        """The float32 value of the softmax scale the kernels use."""
        s = self.softmax_scale if self.softmax_scale is not None else 1.0 / math.sqrt(self.d_qk)
        return float(torch.tensor(s, dtype=torch.float32))

    def c(self) -> _lib.Shape:
        return _lib.Shape(self.batch, self.heads_q, self.heads_kv, self.seqlen, self.d_qk, self.d_v,
                          int(bool(self.causal)), self.sigma)


def padded_len(L: int) -> int:
    return int(_lib.load().dm_padded_len(int(L)))


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _op_shapes(shape: AttnShape, name: str):
    """Expected (codes, scales) shapes of operand ``name`` (q_c, q_s, k_c, k_s, v_c, v_s, do_c, do_s)."""
    B, Lp = shape.batch, padded_len(shape.seqlen)
    H = shape.heads_q if name[0] in "qd" else shape.heads_kv     # Q, dO per query head; K, V per KV head
    d = shape.d_qk if name[0] in "qk" else shape.d_v
    if name.endswith("_c"):
        return (B, H, Lp, d), (B, H, Lp, d // 32)
    return (B, H, d, Lp), (B, H, d, Lp // 32)


def _need_op(shape: AttnShape, op: Fp8Operand, name: str, device) -> None:
    """A quantized operand: GPU, contiguous, uint8 codes and float32 scales of the layout the kernels read."""
    _need(op.codes, name + ".codes", torch.uint8, device)
    _need(op.scales, name + ".scales", torch.float32, device)
    if shape.seqlen > 0:
        cs, ss = _op_shapes(shape, name)
        if tuple(op.codes.shape) != cs or tuple(op.scales.shape) != ss:
            raise ValueError(f"{name}: codes {tuple(op.codes.shape)} / scales {tuple(op.scales.shape)}, "
                             f"expected {cs} / {ss}")


def _need_t(shape: AttnShape, t: Optional[torch.Tensor], name: str, dims, device, dtype=torch.float32) -> None:
    """A dense input or output ([B, H, L] or [B, H, L, d]) of the given dtype, when given."""
    if t is None:
        return
    _need(t, name, dtype, device)
    if shape.seqlen > 0 and tuple(t.shape) != tuple(dims):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(dims)}")


def quantize(x: torch.Tensor, axis: str = "cols", fmt: str = "e4m3", rows_out: Optional[int] = None) -> Fp8Operand:
    """dm_quantize_blockfp8 over the last two dims of x ([..., rows, cols], bf16 or float32).

    axis="cols": codes [..., rows_out, cols], scales [..., rows_out, cols/32].
    axis="rows": codes [..., cols, rows_out], scales [..., cols, rows_out/32] (transposed).
    """
    _need(x, "x")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be bfloat16 or float32")
    *lead, rows, cols = x.shape
    batch = 1
    for n in lead:
        batch *= n
    rows_out = rows if rows_out is None else int(rows_out)
    if axis == "cols":
        codes = torch.empty((*lead, rows_out, cols), dtype=torch.uint8, device=x.device)
        scales = torch.empty((*lead, rows_out, max(cols // 32, 1)), dtype=torch.float32, device=x.device)
    elif axis == "rows":
        codes = torch.empty((*lead, cols, rows_out), dtype=torch.uint8, device=x.device)
        scales = torch.empty((*lead, cols, max(rows_out // 32, 1)), dtype=torch.float32, device=x.device)
    else:
        raise ValueError(f"axis must be 'cols' or 'rows', got {axis!r}")
    dt = _lib.DM_BF16 if x.dtype == torch.bfloat16 else _lib.DM_F32
    st = _lib.load().dm_quantize_blockfp8(x.data_ptr(), dt, batch, rows, cols, rows_out, AXES[axis], FORMATS[fmt],
                                          codes.data_ptr(), scales.data_ptr(), _stream(x))
    _lib.check(st, "dm_quantize_blockfp8")
    return Fp8Operand(codes, scales)


def quantize_operands(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, do: torch.Tensor) -> dict:
    """The eight FP8 operands of the path, padded to dm_padded_len(L).

    X_c: blocks along channels, codes [B, H, Lp, d]; X_s: blocks along the
    sequence, transposed, codes [B, H, d, Lp].
    """
    L = q.shape[-2]
    Lp = padded_len(L)
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v), ("do", do)):
        fmt = OPERAND_FORMAT[name]
        out[name + "_c"] = quantize(x, "cols", fmt, Lp)
        out[name + "_s"] = quantize(x, "rows", fmt, Lp)
    return out


def attn_fwd(shape: AttnShape, q_c: Fp8Operand, k_c: Fp8Operand, v_s: Fp8Operand,
             o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """dm_attn_fwd -> (O [B,Hq,L,d_v] float32, LSE [B,Hq,L] float32)."""
    dev = q_c.codes.device
    B, Hq, L = shape.batch, shape.heads_q, shape.seqlen
    for n, op in (("q_c", q_c), ("k_c", k_c), ("v_s", v_s)):
        _need_op(shape, op, n, dev)
    _need_t(shape, o, "o", (B, Hq, L, shape.d_v), dev)
    _need_t(shape, lse, "lse", (B, Hq, L), dev)
    if o is None:
        o = torch.empty((B, Hq, L, shape.d_v), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    cs = shape.c()
    st = _lib.load().dm_attn_fwd(ctypes.byref(cs), q_c.c(), k_c.c(), v_s.c(), o.data_ptr(), lse.data_ptr(),
                                 _stream(q_c.codes))
    _lib.check(st, "dm_attn_fwd")
    return o, lse


def attn_delta(shape: AttnShape, mode: str, *, o: Optional[torch.Tensor] = None, do: Optional[torch.Tensor] = None,
               do_c: Optional[Fp8Operand] = None, q_c: Optional[Fp8Operand] = None,
               k_c: Optional[Fp8Operand] = None, v_c: Optional[Fp8Operand] = None,
               lse: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dm_attn_delta in mode "stale" (o, do), "do_matched" (o, do_c) or "matched" (do_c, q_c, k_c, v_c, lse)."""
    if mode not in MODES:
        raise ValueError(f"unknown delta mode {mode!r}")
    ref = next(t for t in (o, lse, do, None if do_c is None else do_c.codes) if t is not None)
    dev = ref.device
    B, Hq, L = shape.batch, shape.heads_q, shape.seqlen
    _need_t(shape, o, "o", (B, Hq, L, shape.d_v), dev)
    _need_t(shape, do, "do", (B, Hq, L, shape.d_v), dev, torch.bfloat16)
    _need_t(shape, lse, "lse", (B, Hq, L), dev)
    _need_t(shape, out, "out", (B, Hq, L), dev)
    for n, op in (("do_c", do_c), ("q_c", q_c), ("k_c", k_c), ("v_c", v_c)):
        if op is not None:
            _need_op(shape, op, n, dev)
    if out is None:
        out = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    cs = shape.c()
    opc = lambda x: _NULL_OPERAND if x is None else x.c()  # noqa: E731
    st = _lib.load().dm_attn_delta(ctypes.byref(cs), MODES[mode], _ptr(o), _ptr(do), opc(do_c), opc(q_c),
                                   opc(k_c), opc(v_c), _ptr(lse), out.data_ptr(), _stream(ref))
    _lib.check(st, "dm_attn_delta")
    return out


def _need_bwd(shape: AttnShape, ops: dict, names, lse, delta, dq=None, dk=None, dv=None):
    dev = lse.device
    B, Hq, Hkv, L = shape.batch, shape.heads_q, shape.heads_kv, shape.seqlen
    for n in names:
        _need_op(shape, ops[n], n, dev)
    _need_t(shape, lse, "lse", (B, Hq, L), dev)
    _need_t(shape, delta, "delta", (B, Hq, L), dev)
    _need_t(shape, dq, "dq", (B, Hq, L, shape.d_qk), dev)
    _need_t(shape, dk, "dk", (B, Hkv, L, shape.d_qk), dev)
    _need_t(shape, dv, "dv", (B, Hkv, L, shape.d_v), dev)


def attn_bwd(shape: AttnShape, ops: dict, lse: torch.Tensor, delta: torch.Tensor, probe: bool = False,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None) -> dict:
    """dm_attn_bwd -> {"dq","dk","dv"} float32 (+ "rowsum","rowabs" float64 probes when probe=True)."""
    _need_bwd(shape, ops, ("q_c", "q_s", "k_c", "k_s", "v_c", "do_c", "do_s"), lse, delta, dq, dk, dv)
    dev = lse.device
    B, Hq, Hkv, L = shape.batch, shape.heads_q, shape.heads_kv, shape.seqlen
    if dq is None:
        dq = torch.empty((B, Hq, L, shape.d_qk), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((B, Hkv, L, shape.d_qk), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((B, Hkv, L, shape.d_v), dtype=torch.float32, device=dev)
    ps = pa = None
    if probe:
        ps = torch.empty((B, Hq, L), dtype=torch.float64, device=dev)
        pa = torch.empty((B, Hq, L), dtype=torch.float64, device=dev)
    cs = shape.c()
    st = _lib.load().dm_attn_bwd(ctypes.byref(cs), ops["q_c"].c(), ops["q_s"].c(), ops["k_c"].c(), ops["k_s"].c(),
                                 ops["v_c"].c(), ops["do_c"].c(), ops["do_s"].c(), lse.data_ptr(), delta.data_ptr(),
                                 dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _ptr(ps), _ptr(pa), _stream(lse))
    _lib.check(st, "dm_attn_bwd")
    out = {"dq": dq, "dk": dk, "dv": dv}
    if probe:
        out["rowsum"], out["rowabs"] = ps, pa
    return out


def attn_bwd_dkdv(shape: AttnShape, ops: dict, lse: torch.Tensor, delta: torch.Tensor,
                  dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None, probe: bool = False) -> dict:
    """dm_attn_bwd_dkdv -> {"dk","dv"} float32 (the key-stationary half of dm_attn_bwd).

    With ``probe`` (dm_attn_bwd_dkdv_probes) also "rowsum" and "rowabs" [B,Hq,L] float64: the
    row sums of the dS this kernel casts, before the cast, and of |P dP^|."""
    _need_bwd(shape, ops, ("q_c", "q_s", "k_c", "v_c", "do_c", "do_s"), lse, delta, dk=dk, dv=dv)
    dev = lse.device
    B, Hq, Hkv, L = shape.batch, shape.heads_q, shape.heads_kv, shape.seqlen
    if dk is None:
        dk = torch.empty((B, Hkv, L, shape.d_qk), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((B, Hkv, L, shape.d_v), dtype=torch.float32, device=dev)
    cs = shape.c()
    args = (ctypes.byref(cs), ops["q_c"].c(), ops["q_s"].c(), ops["k_c"].c(), ops["v_c"].c(), ops["do_c"].c(),
            ops["do_s"].c(), lse.data_ptr(), delta.data_ptr(), dk.data_ptr(), dv.data_ptr())
    out = {"dk": dk, "dv": dv}
    if probe:
        ps = torch.empty((B, Hq, L), dtype=torch.float64, device=dev)
        pa = torch.empty((B, Hq, L), dtype=torch.float64, device=dev)
        st = _lib.load().dm_attn_bwd_dkdv_probes(*args, ps.data_ptr(), pa.data_ptr(), _stream(lse))
        _lib.check(st, "dm_attn_bwd_dkdv_probes")
        out["rowsum"], out["rowabs"] = ps, pa
    else:
        st = _lib.load().dm_attn_bwd_dkdv(*args, _stream(lse))
        _lib.check(st, "dm_attn_bwd_dkdv")
    return out


def dkdv_workspace_size(shape: AttnShape) -> int:
    """dm_attn_bwd_dkdv_workspace_size: bytes of workspace ``attn_bwd_dkdv_ws`` needs (0: none)."""
    n = ctypes.c_int64(0)
    cs = shape.c()
    _lib.check(_lib.load().dm_attn_bwd_dkdv_workspace_size(ctypes.byref(cs), ctypes.byref(n)),
               "dm_attn_bwd_dkdv_workspace_size")
    return int(n.value)


def attn_bwd_dkdv_ws(shape: AttnShape, ops: dict, lse: torch.Tensor, delta: torch.Tensor,
                     workspace: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                     dv: Optional[torch.Tensor] = None) -> dict:
    """dm_attn_bwd_dkdv_ws -> {"dk","dv"}: dK/dV with the query heads of a KV group split over
    several workgroups when the grid is small (partial sums in ``workspace``, a device uint8
    tensor of at least ``dkdv_workspace_size(shape)`` bytes; allocated here when None)."""
    _need_bwd(shape, ops, ("q_c", "q_s", "k_c", "v_c", "do_c", "do_s"), lse, delta, dk=dk, dv=dv)
    dev = lse.device
    B, Hkv, L = shape.batch, shape.heads_kv, shape.seqlen
    if dk is None:
        dk = torch.empty((B, Hkv, L, shape.d_qk), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((B, Hkv, L, shape.d_v), dtype=torch.float32, device=dev)
    if workspace is None:
        need = dkdv_workspace_size(shape)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the operands' device")
    wp = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    cs = shape.c()
    st = _lib.load().dm_attn_bwd_dkdv_ws(ctypes.byref(cs), ops["q_c"].c(), ops["q_s"].c(), ops["k_c"].c(),
                                         ops["v_c"].c(), ops["do_c"].c(), ops["do_s"].c(), lse.data_ptr(),
                                         delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), wp, wb, _stream(lse))
    _lib.check(st, "dm_attn_bwd_dkdv_ws")
    return {"dk": dk, "dv": dv}


def attn_bwd_dkdv_noalloc(shape: AttnShape, ops: dict, lse: torch.Tensor, delta: torch.Tensor,
                          dk: torch.Tensor, dv: torch.Tensor) -> dict:
    """dm_attn_bwd_dkdv_noalloc -> {"dk","dv"}: ``attn_bwd_dkdv_ws`` with the library's fixed
    per-device scratch instead of a workspace; the outputs are the caller's (nothing is
    allocated here or in the library).  Calls that overlap on one device race."""
    _need_bwd(shape, ops, ("q_c", "q_s", "k_c", "v_c", "do_c", "do_s"), lse, delta, dk=dk, dv=dv)
    cs = shape.c()
    st = _lib.load().dm_attn_bwd_dkdv_noalloc(ctypes.byref(cs), ops["q_c"].c(), ops["q_s"].c(), ops["k_c"].c(),
                                              ops["v_c"].c(), ops["do_c"].c(), ops["do_s"].c(), lse.data_ptr(),
                                              delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream(lse))
    _lib.check(st, "dm_attn_bwd_dkdv_noalloc")
    return {"dk": dk, "dv": dv}


def attn_bwd_dq(shape: AttnShape, ops: dict, lse: torch.Tensor, delta: torch.Tensor, probe: bool = False,
                dq: Optional[torch.Tensor] = None, probe_cast: bool = False) -> dict:
    """dm_attn_bwd_dq -> {"dq"} float32 (+ "rowsum","rowabs" probes): the query-stationary half.

    With ``probe_cast`` (dm_attn_bwd_dq_probes) also "rowsum_cast": the row sums of dS
    after its E5M2 cast along keys (implies ``probe``)."""
    _need_bwd(shape, ops, ("q_c", "k_c", "k_s", "v_c", "do_c"), lse, delta, dq=dq)
    dev = lse.device
    B, Hq, L = shape.batch, shape.heads_q, shape.seqlen
    if dq is None:
        dq = torch.empty((B, Hq, L, shape.d_qk), dtype=torch.float32, device=dev)
    probe = probe or probe_cast
    ps = pa = pc = None
    if probe:
        ps = torch.empty((B, Hq, L), dtype=torch.float64, device=dev)
        pa = torch.empty((B, Hq, L), dtype=torch.float64, device=dev)
    cs = shape.c()
    args = (ctypes.byref(cs), ops["q_c"].c(), ops["k_c"].c(), ops["k_s"].c(), ops["v_c"].c(), ops["do_c"].c(),
            lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), _ptr(ps), _ptr(pa))
    if probe_cast:
        pc = torch.empty((B, Hq, L), dtype=torch.float64, device=dev)
        st = _lib.load().dm_attn_bwd_dq_probes(*args, _ptr(pc), _stream(lse))
        _lib.check(st, "dm_attn_bwd_dq_probes")
    else:
        st = _lib.load().dm_attn_bwd_dq(*args, _stream(lse))
        _lib.check(st, "dm_attn_bwd_dq")
    out = {"dq": dq}
    if probe:
        out["rowsum"], out["rowabs"] = ps, pa
    if probe_cast:
        out["rowsum_cast"] = pc
    return out


def fwd_delta_bwd(shape: AttnShape, ops: dict, mode: str = "matched", do: Optional[torch.Tensor] = None,
                  probe: bool = False, split: bool = False) -> dict:
    """One pass of the whole path on already-quantized operands: forward, delta, backward.

    ``split``: the backward as dm_attn_bwd_dkdv_ws (head split of small grids, workspace
    allocated here) plus dm_attn_bwd_dq instead of the fused dm_attn_bwd."""
    o, lse = attn_fwd(shape, ops["q_c"], ops["k_c"], ops["v_s"])
    if mode == "matched":
        d = attn_delta(shape, mode, do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"], v_c=ops["v_c"], lse=lse)
    elif mode == "do_matched":
        d = attn_delta(shape, mode, o=o, do_c=ops["do_c"])
    else:
        d = attn_delta(shape, mode, o=o, do=do)
    if split and not probe:
        g = attn_bwd_dkdv_ws(shape, ops, lse, d)
        g.update(attn_bwd_dq(shape, ops, lse, d))
    else:
        g = attn_bwd(shape, ops, lse, d, probe=probe)
    g.update(o=o, lse=lse, delta=d)
    return g
