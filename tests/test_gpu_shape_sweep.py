"""GPU parity on a seeded sweep of small random shapes (run with ``-m gpu`` on an MI355X).

The fixed cases elsewhere pick shapes by hand; this sweep draws batch, query-group
size (GQA up to 16 query heads per KV head), KV heads, length (ragged, one-token,
exact multiples of the tiles), every supported head-dimension pair, the causal
flag, the input family and sometimes an explicit softmax scale, all from one seed,
and checks the whole matched chain -- forward (O, LSE), matched delta, dQ, dK, dV
on the instances the benchmark runs -- plus the head-split dK/dV entry
(dm_attn_bwd_dkdv_ws) against the oracle, with the bars of the other parity tests, and
the allocation-free entry (dm_attn_bwd_dkdv_noalloc) bit for bit against it.
"""
import sys

import numpy as np
import pytest
import torch

from fp8_attention_amd import workloads as W
from oracle import attention as A
from tests import parity_util as U

pytestmark = pytest.mark.gpu

DIMS = [(128, 128)] * 4 + [(64, 64), (192, 128), (64, 128), (128, 64), (192, 64), (256, 256)]
KINDS = ["rmsnorm", "iid", "scaled"]
N_CASES = 64


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _draw(n: int):
    """n shapes from one seed; the oracle's cost B*Hq*L*L*d is capped so each case takes seconds."""
    rng = np.random.RandomState(20261202)
    out = []
    while len(out) < n:
        d_qk, d_v = DIMS[rng.randint(len(DIMS))]
        hkv = int(rng.randint(1, 4))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        b = int(rng.randint(1, 4))
        r = rng.rand()
        if r < 0.15:
            L = int(rng.choice([1, 2, 31, 33]))
        elif r < 0.35:
            L = int(rng.choice([127, 128, 129, 255, 256, 257, 384]))
        else:
            L = int(rng.randint(3, 420))
        if b * g * hkv * L * L * (d_qk + d_v) > 6e8:
            continue
        causal = bool(rng.rand() < 0.7)
        kind = KINDS[rng.randint(len(KINDS))]
        sigma = float(rng.uniform(0.03, 0.4)) if rng.rand() < 0.25 else None
        i = len(out)
        name = f"s{i:02d}_b{b}_h{g * hkv}x{hkv}_L{L}_d{d_qk}x{d_v}_{'c' if causal else 'nc'}_{kind}"
        out.append((name, W.small(name, batch=b, heads_q=g * hkv, heads_kv=hkv, seqlen=L, d_qk=d_qk, d_v=d_v,
                                  causal=causal, kind=kind, seed=3000 + i), sigma))
    return out


CASES = _draw(N_CASES)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sweep_chain_and_head_split(case):
    from fp8_attention_amd import api
    name, w, scale = case
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal, scale)
    shp = U.oracle_shape(w, shape.sigma)
    inputs = W.generate(w)
    _log(f"[sweep] {name} sigma={shape.sigma:.4f} head-split workspace {api.dkdv_workspace_size(shape)} B")
    ref = U.run_oracle(inputs, shp, modes=("matched",))
    dev = {n: t.cuda() for n, t in inputs.items()}
    ops = api.quantize_operands(dev["q"], dev["k"], dev["v"], dev["do"])
    g = api.fwd_delta_bwd(shape, ops, "matched")
    split = api.attn_bwd_dkdv_ws(shape, ops, g["lse"], g["delta"])
    # the allocation-free entry: same kernels on the library's fixed scratch, same bits
    na = {"dk": torch.empty_like(split["dk"]), "dv": torch.empty_like(split["dv"])}
    api.attn_bwd_dkdv_noalloc(shape, ops, g["lse"], g["delta"], na["dk"], na["dv"])
    torch.cuda.synchronize()
    assert torch.equal(na["dk"], split["dk"]) and torch.equal(na["dv"], split["dv"])
    f, r = ref["fwd"], ref["matched"]
    U.compare("O", g["o"], f["o"], allow=f["r_o"] + f["b_o"], norm_rel=U.NORM_TOL, flip=f["r_o"])
    U.compare("LSE", g["lse"], f["lse"], allow=f["b_lse"], rel=0.0)
    derr = A.delta_bound(ref["ops"], shp, "matched", lse=f["lse"], lse_err=f["b_lse"])
    U.compare("delta", g["delta"], r["delta"], allow=derr, rel=0.0)
    b = A.backward(ref["ops"], shp, f["lse"], r["delta"], radius=True, delta_err=derr, lse_err=f["b_lse"])
    for n in ("dq", "dk", "dv"):
        _log("   ", U.compare(n, g[n], b[n], allow=b["r_" + n] + b["b_" + n], norm_rel=U.NORM_TOL, flip=b["r_" + n]))
    for n in ("dk", "dv"):
        _log("   ", U.compare(n + " (head split)", split[n], b[n], allow=b["r_" + n] + b["b_" + n],
                              norm_rel=U.NORM_TOL, flip=b["r_" + n]))
    if api.dkdv_workspace_size(shape) == 0:
        assert torch.equal(split["dk"], g["dk"]) and torch.equal(split["dv"], g["dv"])
