"""The allocation-free dK/dV entry point (dm_attn_bwd_dkdv_noalloc) against the workspace
entry point it varies (dm_attn_bwd_dkdv_ws): same kernels, same head split, so dK and dV
must agree bit for bit.  Two calls in a row, the second on a smaller problem, so the
second runs on a scratch that still holds the first call's partial sums.
"""
import sys

import pytest
import torch

from fp8_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _problem(w):
    from fp8_attention_amd import api
    inputs = W.generate(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal)
    ops = api.quantize_operands(dev["q"], dev["k"], dev["v"], dev["do"])
    _, lse = api.attn_fwd(shape, ops["q_c"], ops["k_c"], ops["v_s"])
    delta = api.attn_delta(shape, "matched", do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"], v_c=ops["v_c"],
                           lse=lse)
    return shape, ops, lse, delta


def test_noalloc_matches_workspace_entry_on_two_calls():
    from fp8_attention_amd import _lib, api
    cases = [
        # the 4K GQA workload: heads split over 4 workgroups per key tile, the whole scratch
        W.WORKLOADS["gqa_4k"],
        # a smaller, ragged multi-query problem: split over 8, a small part of the scratch
        W.small("mqa_ragged", batch=1, heads_q=8, heads_kv=1, seqlen=200, d_qk=128, d_v=128, causal=True,
                kind="rmsnorm", seed=31),
    ]
    for w in cases:
        _log(f"[noalloc] {w.name}")
        shape, ops, lse, delta = _problem(w)
        need = api.dkdv_workspace_size(shape)
        assert 0 < need <= _lib.DM_NOALLOC_SCRATCH_BYTES, need
        dk = torch.empty((w.batch, w.heads_kv, w.seqlen, w.d_qk), dtype=torch.float32, device="cuda")
        dv = torch.empty((w.batch, w.heads_kv, w.seqlen, w.d_v), dtype=torch.float32, device="cuda")
        api.attn_bwd_dkdv_noalloc(shape, ops, lse, delta, dk, dv)
        ref = api.attn_bwd_dkdv_ws(shape, ops, lse, delta)
        torch.cuda.synchronize()
        assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
        assert torch.equal(dk, ref["dk"]), f"{w.name}: dK differs from the workspace entry point's"
        assert torch.equal(dv, ref["dv"]), f"{w.name}: dV differs from the workspace entry point's"
        _log(f"   {need} bytes of scratch; dK, dV bit-identical to the workspace entry point")
