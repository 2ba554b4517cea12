"""Seeded synthetic attention workloads (inputs only).

This module draws the bf16 tensors Q, K, V and dO that both the HIP path and
the CPU oracle consume.  It holds none of the attention method's arithmetic:
it only samples Gaussians, applies the per-head RMSNorm that makes Q and K look
like the normalised projections the Delta-Matching project page trains with
("QK normalization", section 05, and the channel-gain diagnostics of section
02), and rounds to bf16.

Recipe (one generator per workload, seeded with ``1000 + index``):
  * draws happen in the order Q, K, V, dO, each a full-shape float32 standard
    normal tensor of logical layout [B, H, L, d];
  * ``iid``   : Q, K, V, dO ~ N(0, 1);
  * ``rmsnorm``: Q and K are normalised over d (eps 1e-6, float32), then
    multiplied by per-channel gains (1.0 unless overridden), V ~ N(0, 1),
    dO ~ N(0, 1e-2) (variance 1e-2, i.e. std 0.1);
  * ``scaled``: Q, K ~ N(0, 1) / sqrt(d_qk), V ~ N(0, 1), dO ~ N(0, 1e-2);
  * everything is finally rounded to bf16 (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    d_qk: int
    d_v: int
    causal: bool
    kind: str = "iid"            # "iid" | "rmsnorm" | "scaled"
    q_gain7: float = 1.0         # RMSNorm gain on channel 7 of Q
    k_gain7: float = 1.0         # RMSNorm gain on channel 7 of K
    seed: int = 1000

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def matmul_flops(self) -> float:
        """Seven-matmul FLOP count: 2*(4*d_qk + 3*d_v) per (query, key) pair and head,
        with L^2/2 pairs when causal and L^2 otherwise."""
        pairs = self.seqlen * self.seqlen / (2.0 if self.causal else 1.0)
        return 2.0 * (4 * self.d_qk + 3 * self.d_v) * pairs * self.batch * self.heads_q


# The five synthetic workloads: a tiny single head, a GQA layer, the long-context
# GQA layer with near-saturated rows (channel-7 gains 2.0 on Q and 5.4 on K, the
# key gain the project page reports for stale delta), the 64K context-extension
# shape, and an MLA-shaped layer with d_qk = 192, d_v = 128; plus the GQA layer at
# head dimension 256, the head geometry of the project page's larger models.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 128, 64, 64, False, "iid", seed=1000),
    "gqa_4k": Workload("gqa_4k", 2, 16, 4, 4096, 128, 128, True, "rmsnorm", seed=1001),
    "gqa_8k": Workload("gqa_8k", 4, 32, 8, 8192, 128, 128, True, "rmsnorm",
                       q_gain7=2.0, k_gain7=5.4, seed=1002),
    "gqa_64k": Workload("gqa_64k", 1, 16, 4, 65536, 128, 128, True, "rmsnorm", seed=1003),
    "mla_4k": Workload("mla_4k", 2, 16, 16, 4096, 192, 128, True, "scaled", seed=1004),
    "gqa_d256_4k": Workload("gqa_d256_4k", 2, 16, 4, 4096, 256, 256, True, "rmsnorm", seed=1005),
}


def _rmsnorm(x: torch.Tensor, gain7: float) -> torch.Tensor:
    y = x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + 1e-6)
    if gain7 != 1.0 and y.shape[-1] > 7:
        g = torch.ones(y.shape[-1], dtype=y.dtype)
        g[7] = gain7
        y = y * g
    return y


def generate(w: Workload, device: Optional[str] = None) -> dict:
    """Return {"q","k","v","do"} as bf16 CPU tensors of shape [B, H, L, d]."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    B, Hq, Hkv, L = w.batch, w.heads_q, w.heads_kv, w.seqlen
    q = torch.randn((B, Hq, L, w.d_qk), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, L, w.d_qk), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, L, w.d_v), generator=g, dtype=torch.float32)
    do = torch.randn((B, Hq, L, w.d_v), generator=g, dtype=torch.float32)
    if w.kind == "rmsnorm":
        q = _rmsnorm(q, w.q_gain7)
        k = _rmsnorm(k, w.k_gain7)
        do = do * 0.1
    elif w.kind == "scaled":
        q = q / math.sqrt(w.d_qk)
        k = k / math.sqrt(w.d_qk)
        do = do * 0.1
    elif w.kind != "iid":
        raise ValueError(f"unknown workload kind {w.kind!r}")
    out = {n: t.to(torch.bfloat16) for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}
    if device is not None:
        out = {n: t.to(device) for n, t in out.items()}
    return out


def small(name: str = "small", *, batch=1, heads_q=2, heads_kv=1, seqlen=320, d_qk=64, d_v=64,
          causal=True, kind="rmsnorm", q_gain7=1.0, k_gain7=1.0, seed=7) -> Workload:
    """A reduced workload for parity tests (several tiles plus a ragged tail)."""
    return Workload(name, batch, heads_q, heads_kv, seqlen, d_qk, d_v, causal, kind, q_gain7, k_gain7, seed)
