"""The autograd entry (fp8_attention_amd.autograd) and a synthetic logit-drift demo.

CPU: argument validation (nothing reaches the library).
GPU: the wrapper's output and gradients are bit-identical to the direct call
chain (quantize, forward, delta, backward), which the oracle parity tests cover;
the wrapper agrees with float64 attention to within FP8 quantization error; and
the drift demo of the Delta-Matching page, section 02 ("What does stale delta
do to training?"): stale delta adds eps_i P_ij to every dS row
(eps_i = delta_matched_i - delta_stale_i), and a small gradient step on the
logits along -eps_i P_i changes the row entropy by
    eta * eps_i * sum_j P_ij^2 (log P_ij + H_i)  (= eta eps_i Cov_P(P, log P) >= 0 for eps_i > 0),
i.e. flattens the row when eps_i > 0 and sharpens it when eps_i < 0.
"""
import sys

import numpy as np
import pytest
import torch

from fp8_attention_amd import autograd as AG


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- CPU: validation

def _qkv(B=1, Hq=2, Hkv=1, L=64, dqk=64, dv=64, dtype=torch.bfloat16, device="cpu"):
    g = torch.Generator().manual_seed(3)
    mk = lambda *s: torch.randn(*s, generator=g).to(dtype).to(device)   # noqa: E731
    return mk(B, Hq, L, dqk), mk(B, Hkv, L, dqk), mk(B, Hkv, L, dv)


def test_check_inputs_accepts_gqa_shapes():
    q, k, v = _qkv(Hq=4, Hkv=2, dv=128)
    s = AG.check_inputs(q, k, v, "matched")
    assert (s.batch, s.heads_q, s.heads_kv, s.seqlen, s.d_qk, s.d_v) == (1, 4, 2, 64, 64, 128)


@pytest.mark.parametrize("case", ["mode", "rank", "dtype", "mixed", "contig", "group", "len", "vheads"])
def test_check_inputs_rejects(case):
    q, k, v = _qkv()
    mode = "matched"
    if case == "mode":
        mode = "centered"
    elif case == "rank":
        q = q[0]
    elif case == "dtype":
        q, k, v = q.half(), k.half(), v.half()
    elif case == "mixed":
        q = q.float()
    elif case == "contig":
        q = q.transpose(2, 3)
    elif case == "group":
        q = torch.cat([q, q[:, :1]], dim=1)        # 3 query heads over 2 KV heads
        k = torch.cat([k, k], dim=1)
        v = torch.cat([v, v], dim=1)
    elif case == "len":
        k = k[:, :, :32].contiguous()
    elif case == "vheads":
        v = torch.cat([v, v], dim=1)
    with pytest.raises(ValueError):
        AG.check_inputs(q, k, v, mode)


# ---------------------------------------------------------------- GPU

CHAIN_CASES = [
    # (B, Hq, Hkv, L, dqk, dv, causal, mode, dtype)
    (1, 2, 1, 200, 128, 128, True, "matched", torch.bfloat16),
    (2, 4, 2, 129, 64, 64, False, "stale", torch.bfloat16),
    (1, 2, 2, 257, 192, 128, True, "do_matched", torch.bfloat16),
    (1, 4, 1, 320, 128, 128, True, "matched", torch.float32),
    (1, 2, 1, 129, 256, 256, True, "matched", torch.bfloat16),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CHAIN_CASES, ids=lambda c: f"L{c[3]}-d{c[4]}x{c[5]}-{c[7]}-{str(c[8])[6:]}")
def test_autograd_matches_call_chain(case):
    from fp8_attention_amd import api
    B, Hq, Hkv, L, dqk, dv, causal, mode, dtype = case
    q, k, v = (t.cuda() for t in _qkv(B, Hq, Hkv, L, dqk, dv, dtype))
    do = (0.1 * torch.randn(B, Hq, L, dv, generator=torch.Generator().manual_seed(5))).to(torch.bfloat16).cuda()
    qr, kr, vr = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = AG.fp8_attention(qr, kr, vr, causal=causal, delta_mode=mode)
    o.backward(do.to(o.dtype))
    # the same steps through the binding
    shape = api.AttnShape(B, Hq, Hkv, L, dqk, dv, causal)
    ops = api.quantize_operands(q, k, v, do)
    g = api.fwd_delta_bwd(shape, ops, mode=mode, do=do, split=True)
    torch.cuda.synchronize()
    assert o.dtype == dtype and qr.grad.dtype == dtype
    assert torch.equal(o, g["o"].to(dtype))
    for n, t in (("dq", qr), ("dk", kr), ("dv", vr)):
        assert torch.equal(t.grad, g[n].to(dtype)), n


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
def test_autograd_close_to_float64_attention(causal):
    """A drop-in check: FP8 attention and its gradients against float64 attention
    (CPU autograd, GQA by repeating the KV heads) to within FP8 quantization error,
    measured as relative Frobenius error."""
    B, Hq, Hkv, L, d = 1, 4, 2, 256, 128
    q, k, v = _qkv(B, Hq, Hkv, L, d, d, torch.bfloat16)
    do = (0.1 * torch.randn(B, Hq, L, d, generator=torch.Generator().manual_seed(9))).to(torch.bfloat16)
    qr, kr, vr = (t.cuda().requires_grad_(True) for t in (q, k, v))
    o = AG.fp8_attention(qr, kr, vr, causal=causal)
    o.backward(do.cuda())
    q64, k64, v64 = (t.double().requires_grad_(True) for t in (q, k, v))
    G = Hq // Hkv
    s = (q64 @ k64.repeat_interleave(G, 1).transpose(-1, -2)) / d ** 0.5
    if causal:
        s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
    o64 = torch.softmax(s, -1) @ v64.repeat_interleave(G, 1)
    o64.backward(do.double())
    rel = lambda a, b: float((a.double().cpu() - b).norm() / b.norm())   # noqa: E731
    errs = {"o": rel(o.detach(), o64.detach()), "dq": rel(qr.grad, q64.grad), "dk": rel(kr.grad, k64.grad),
            "dv": rel(vr.grad, v64.grad)}
    _log("   relative error vs float64:", {n: f"{e:.3e}" for n, e in errs.items()})
    # RNE to 3 (E4M3) or 2 (E5M2) mantissa bits leaves a relative error uniform within
    # +-2^-4 or +-2^-3 per element, RMS r4 = 2^-4/sqrt(3) ~ 3.6% or r5 = 2^-3/sqrt(3) ~ 7.2%.
    # On these zero-mean operands the errors of a product's terms add up like its values, so
    # the relative error of a product is about the root-sum-square of its operands' r:
    # O = P^ V^: sqrt(2) r4 ~ 5.1%; dV = P^T dO^: ~8.1%; dQ, dK (dS from dO^, V^, then E5M2,
    # times K^ or Q^): sqrt(2 r5^2 + 2 r4^2) ~ 11%.  Bars: 1.5x these estimates.
    assert errs["o"] < 0.08 and errs["dv"] < 0.12
    assert errs["dq"] < 0.17 and errs["dk"] < 0.17


def _entropy_terms(q, k, sigma):
    """float64 row entropy H_i and c_i = sum_j P_ij^2 (log P_ij + H_i) of softmax(sigma q k^T)."""
    s = sigma * (q.double() @ k.double().transpose(-1, -2))
    lp = torch.log_softmax(s, -1)
    p = lp.exp()
    h = -(p * lp).sum(-1)
    c = (p * p * (lp + h[..., None])).sum(-1)
    return h, c


@pytest.mark.gpu
def test_logit_drift_stale_vs_matched():
    """Gradient steps on one layer's logits under stale and matched delta.

    The keys of each head are alpha times an orthonormal basis (L = d), so with K
    fixed a step on Q is a step on the logits: S = sigma Q K^T changes by
    -eta sigma dQ K^T = -eta sigma^2 dS^ K^<s> K^T ~ -eta dS^ (sigma^2 alpha^2 = 1).
    One step from the same Q: the entropy difference stale - matched of each row
    follows the first-order prediction eta eps_i c_i (c_i >= 0); T steps: each run
    follows its own Q, and the accumulated difference follows the accumulated
    prediction of the stale run."""
    from fp8_attention_amd import api
    H, L, d = 64, 128, 128
    g = torch.Generator().manual_seed(11)
    alpha = d ** 0.5
    basis = torch.linalg.qr(torch.randn(H, d, d, generator=g, dtype=torch.float64)).Q.transpose(-1, -2)
    k = (alpha * basis).float()[None].contiguous().cuda()               # rows orthogonal, norm sqrt(d)
    q0 = (2.5 * torch.randn(1, H, L, d, generator=g)).cuda()            # logits ~ N(0, 2.5^2)
    v = torch.randn(1, H, L, d, generator=g).cuda()
    do = (0.1 * torch.randn(1, H, L, d, generator=g)).to(torch.bfloat16).cuda()
    sigma = 1.0 / d ** 0.5
    eta = 0.1
    shape = api.AttnShape(1, H, H, L, d, d, False)

    def eps_of(q):
        ops = api.quantize_operands(q, k, v, do)
        o, lse = api.attn_fwd(shape, ops["q_c"], ops["k_c"], ops["v_s"])
        dm = api.attn_delta(shape, "matched", do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"], v_c=ops["v_c"],
                            lse=lse)
        ds = api.attn_delta(shape, "stale", o=o, do=do)
        return (dm - ds).double()

    def step(q, mode):
        qr = q.clone().requires_grad_(True)
        AG.fp8_attention(qr, k, v, delta_mode=mode).backward(do.float())
        return (q - eta * qr.grad).detach()

    # one step from the same point
    h0, c0 = _entropy_terms(q0, k, sigma)
    eps0 = eps_of(q0)
    hs, _ = _entropy_terms(step(q0, "stale"), k, sigma)
    hm, _ = _entropy_terms(step(q0, "matched"), k, sigma)
    diff = (hs - hm).flatten().cpu().numpy()
    pred = (eta * eps0 * c0).flatten().cpu().numpy()
    r1 = float(np.corrcoef(pred, diff)[0, 1])
    slope1 = float(pred @ diff / (pred @ pred))
    top = np.abs(pred) >= np.quantile(np.abs(pred), 0.75)
    agree1 = float(np.mean(np.sign(pred[top]) == np.sign(diff[top])))
    _log(f"   one step: corr(pred, H_stale - H_matched) = {r1:.3f}, slope {slope1:.3f}, "
         f"sign agreement on the top quarter |pred| {agree1:.3f}; mean |eps| {float(eps0.abs().mean()):.3e}")

    # T steps, each mode on its own trajectory
    T = 10
    qs, qm = q0.clone(), q0.clone()
    acc = torch.zeros_like(h0)
    for _ in range(T):
        _, cs = _entropy_terms(qs, k, sigma)
        acc += eta * eps_of(qs) * cs
        qs, qm = step(qs, "stale"), step(qm, "matched")
    hsT, _ = _entropy_terms(qs, k, sigma)
    hmT, _ = _entropy_terms(qm, k, sigma)
    diffT = (hsT - hmT).flatten().cpu().numpy()
    predT = acc.flatten().cpu().numpy()
    rT = float(np.corrcoef(predT, diffT)[0, 1])
    sharp = predT < np.quantile(predT, 0.25)        # rows pushed hardest toward sharpening
    flat = predT > np.quantile(predT, 0.75)
    _log(f"   {T} steps: corr(accumulated pred, H_stale - H_matched) = {rT:.3f}; mean entropy difference "
         f"{float(diffT[sharp].mean()):.3e} on the quarter pushed to sharpen, "
         f"{float(diffT[flat].mean()):.3e} on the quarter pushed to flatten")
    # first order predicts slope 1; the E5M2 cast of dS adds noise around it
    assert r1 > 0.5 and 0.5 < slope1 < 1.5
    assert rT > 0.5
    assert diffT[sharp].mean() < 0 < diffT[flat].mean()
