"""GPU parity of libdm against the CPU oracle (run with ``-m gpu`` on an MI355X).

Bar (per tensor): FP8 codes and scales bit-exact.  O, dQ, dK, dV: norm-wise
||gpu - oracle|| <= 2e-3 ||oracle||, and elementwise |gpu - oracle| <=
2e-3 RMS(oracle) + allowance, where the allowance is the oracle's bound of
(a) the FP8 matrix cores' own accumulation error on that output and (b) the
first-order radius of in-kernel casts whose exact input lies within the
kernel's error budget of a rounding or scale boundary (both casts are correct
there).  LSE and delta within their error bounds.  Under Delta-Matching
|sum_j dS_ij| <= 1e-5 sum_j |P_ij dP_ij| on the kernel's own pre-cast dS, for the
dS of both backward kernels (dQ and dK/dV).

The probing instances of the two backward kernels run the arithmetic of the timed
ones: wherever a test uses the probes it also runs the timed instances and
requires bit-identical dQ, dK and dV, so every comparison below covers the
kernels bench.py times.
"""
import functools
import sys

import numpy as np
import pytest
import torch

from fp8_attention_amd import workloads as W
from oracle import attention as A
from oracle import fp8
from tests import parity_util as U

pytestmark = pytest.mark.gpu

MODES = ("stale", "do_matched", "matched")


def _api():
    from fp8_attention_amd import api
    return api


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


SMALL = {
    # the tiny single-head workload exactly
    "tiny": W.WORKLOADS["tiny"],
    # GQA, causal, ragged length (2.5 tiles), RMSNorm'd Q/K
    "gqa_ragged": W.small("gqa_ragged", batch=2, heads_q=4, heads_kv=2, seqlen=320, d_qk=128, d_v=128,
                          causal=True, kind="rmsnorm", seed=11),
    # near-saturated rows (channel-7 gains of the long-context workload)
    "gqa_gain": W.small("gqa_gain", batch=1, heads_q=4, heads_kv=1, seqlen=384, d_qk=128, d_v=128, causal=True,
                        kind="rmsnorm", q_gain7=2.0, k_gain7=5.4, seed=12),
    # MLA-shaped head dims
    "mla": W.small("mla", batch=1, heads_q=2, heads_kv=2, seqlen=200, d_qk=192, d_v=128, causal=True,
                   kind="scaled", seed=13),
    # non-causal, mixed head dims, ragged
    "mixed_nc": W.small("mixed_nc", batch=1, heads_q=2, heads_kv=1, seqlen=257, d_qk=64, d_v=128, causal=False,
                        kind="iid", seed=14),
    # head dimension 256: GQA, causal, ragged (several 64-key dQ chunks, two 128-query tiles)
    "d256": W.small("d256", batch=1, heads_q=4, heads_kv=2, seqlen=200, d_qk=256, d_v=256, causal=True,
                    kind="rmsnorm", seed=15),
    # head dimension 256, non-causal, iid, one key past a 128 boundary
    "d256_nc": W.small("d256_nc", batch=1, heads_q=2, heads_kv=1, seqlen=129, d_qk=256, d_v=256, causal=False,
                       kind="iid", seed=16),
}


@functools.lru_cache(maxsize=None)
def _case(name):
    w = SMALL[name]
    inputs = W.generate(w)
    api = _api()
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal)
    shp = U.oracle_shape(w, shape.sigma)
    _log(f"[oracle] {name}")
    ref = U.run_oracle(inputs, shp, modes=MODES)
    return w, inputs, shape, shp, ref


def _gpu_ops(inputs):
    api = _api()
    dev = {n: t.cuda() for n, t in inputs.items()}
    return dev, api.quantize_operands(dev["q"], dev["k"], dev["v"], dev["do"])


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _timed_instances_and_dkdv_probes(shape, ops, lse, delta, g):
    """Run the timed (probe-free) backward instances on the same inputs as the probing call
    ``g`` and require its exact bits; return the dK/dV kernel's own row-sum probes."""
    api = _api()
    plain = api.attn_bwd_dq(shape, ops, lse, delta)
    pk = api.attn_bwd_dkdv(shape, ops, lse, delta, probe=True)
    torch.cuda.synchronize()
    assert torch.equal(plain["dq"], g["dq"]), "probing dQ instance differs from the timed one"
    assert torch.equal(pk["dk"], g["dk"]) and torch.equal(pk["dv"], g["dv"]), \
        "probing dK/dV instance differs from the timed one"
    return pk


def _assert_zero_rowsums(p, what):
    rs, ra = U.to64(p["rowsum"]), U.to64(p["rowabs"])
    ratio = np.abs(rs) / np.maximum(ra, 1e-300)
    _log(f"   {what}: max |sum_j dS_ij| / sum_j |P dP| = {float(ratio.max()):.2e}")
    assert np.all(np.abs(rs) <= U.ROWSUM_TOL * ra), (what, float(ratio.max()))


# ---------------------------------------------------------------------------
# quantize: bit-exact codes and scales
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(SMALL))
def test_quantize_operands_bit_exact(name):
    w, inputs, shape, shp, ref = _case(name)
    _log(f"[quantize] {name}")
    _, ops = _gpu_ops(inputs)
    torch.cuda.synchronize()
    L, Lp = w.seqlen, _api().padded_len(w.seqlen)
    L32 = (L + 31) // 32 * 32
    for key, (codes, scales) in ref["qops"].items():
        g = ops[key]
        gc, gs = g.codes.cpu().numpy(), g.scales.cpu().numpy().astype(np.float64)
        if key.endswith("_c"):
            assert np.array_equal(gc[..., :L, :], codes), key
            assert np.array_equal(gs[..., :L, :], scales), key
            assert not gc[..., L:, :].any() and np.all(gs[..., L:, :] == 2.0 ** -126), key
        else:
            assert np.array_equal(gc[..., :L32], codes), key
            assert np.array_equal(gs[..., :L32 // 32], scales), key
            assert not gc[..., L32:].any() and np.all(gs[..., L32 // 32:] == 2.0 ** -126), key
    assert Lp % 128 == 0 and Lp >= L


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("axis", ["cols", "rows"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_special_values(fmt, axis, dtype):
    """Zeros, bf16 subnormals, huge and tiny blocks, exact scale boundaries, negative zero."""
    api = _api()
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 96, 64)) * np.exp(rng.uniform(-30, 30, (3, 96, 1)))
    x[0, :32] = 0.0                                     # all-zero blocks
    x[0, 32:40] = -0.0
    x[1, :8] = 1e-40                                    # subnormal in bf16/f32
    x[1, 8:16, :32] = fp8.FORMATS[fmt].fmax * 2.0 ** 5  # amax exactly on a boundary
    x[2, :4] = 3e38 if dtype == torch.float32 else 1e38
    xt = torch.from_numpy(x).to(dtype)
    xd = xt.double().numpy()
    rows_out = 128
    got = api.quantize(xt.cuda(), axis, fmt, rows_out)
    torch.cuda.synchronize()
    if axis == "cols":
        xp = np.zeros((3, rows_out, 64))
        xp[:, :96] = xd
        codes, scales, _ = fp8.quantize_lastaxis(xp, fmt)
    else:
        xp = np.zeros((3, 64, rows_out))
        xp[:, :, :96] = np.swapaxes(xd, 1, 2)
        codes, scales, _ = fp8.quantize_lastaxis(xp, fmt)
    assert np.array_equal(got.codes.cpu().numpy(), codes)
    assert np.array_equal(got.scales.cpu().numpy().astype(np.float64), scales)


# ---------------------------------------------------------------------------
# forward, delta, backward, each against the oracle with the oracle's own upstream values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(SMALL))
def test_fwd_parity(name):
    w, inputs, shape, shp, ref = _case(name)
    _log(f"[fwd] {name}")
    api = _api()
    _, ops = _gpu_ops(inputs)
    o, lse = api.attn_fwd(shape, ops["q_c"], ops["k_c"], ops["v_s"])
    torch.cuda.synchronize()
    f = ref["fwd"]
    s = U.compare("O", o, f["o"], allow=f["r_o"] + f["b_o"], norm_rel=U.NORM_TOL, flip=f["r_o"])
    U.compare("LSE", lse, f["lse"], allow=f["b_lse"], rel=0.0)
    _log(f"   {s} flagged casts {f['n_flag']} blocks {f['n_block_flag']}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", list(SMALL))
def test_delta_parity(name, mode):
    w, inputs, shape, shp, ref = _case(name)
    _log(f"[delta] {name} {mode}")
    api = _api()
    dev, ops = _gpu_ops(inputs)
    f = ref["fwd"]
    o32, lse32 = _f32(f["o"]), _f32(f["lse"])
    d = api.attn_delta(shape, mode, o=o32, do=dev["do"], do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"],
                       v_c=ops["v_c"], lse=lse32)
    torch.cuda.synchronize()
    want = ref[mode]["delta"]
    tol = A.delta_bound(ref["ops"], shp, mode, o=f["o"], do=ref["do"], lse=f["lse"])
    U.compare("delta", d, want, allow=tol + 1e-30, rel=0.0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", list(SMALL))
def test_bwd_parity(name, mode):
    w, inputs, shape, shp, ref = _case(name)
    _log(f"[bwd] {name} {mode}")
    api = _api()
    _, ops = _gpu_ops(inputs)
    r = ref[mode]
    lse32, d32 = _f32(ref["fwd"]["lse"]), _f32(r["delta"])
    g = api.attn_bwd(shape, ops, lse32, d32, probe=True)
    torch.cuda.synchronize()
    pk = _timed_instances_and_dkdv_probes(shape, ops, lse32, d32, g)
    b = r["bwd"]
    for n in ("dq", "dk", "dv"):
        s = U.compare(n, g[n], b[n], allow=b["r_" + n] + b["b_" + n], norm_rel=U.NORM_TOL, flip=b["r_" + n])
        _log(f"   {s}")
    # both kernels' pre-cast row sums follow the oracle's within the kernel's error bound
    for who, p in (("dq", g), ("dkdv", pk)):
        U.compare(who + " rowsum", p["rowsum"], b["rowsum"], allow=b["b_rowsum"] + 1e-30, rel=0.0)
        U.compare(who + " rowabs", p["rowabs"], b["rowabs"], allow=b["b_rowsum"] + 1e-30, rel=0.0)


@pytest.mark.parametrize("name", list(SMALL))
def test_chain_matched_rowsums_and_parity(name):
    """The benchmarked chain (fwd -> matched delta -> bwd) entirely on the GPU."""
    w, inputs, shape, shp, ref = _case(name)
    _log(f"[chain matched] {name}")
    api = _api()
    _, ops = _gpu_ops(inputs)
    g = api.fwd_delta_bwd(shape, ops, "matched", probe=True)
    torch.cuda.synchronize()
    f, r = ref["fwd"], ref["matched"]
    U.compare("O", g["o"], f["o"], allow=f["r_o"] + f["b_o"], norm_rel=U.NORM_TOL, flip=f["r_o"])
    derr = A.delta_bound(ref["ops"], shp, "matched", lse=f["lse"], lse_err=f["b_lse"])
    U.compare("delta", g["delta"], r["delta"], allow=derr, rel=0.0)
    b = A.backward(ref["ops"], shp, f["lse"], r["delta"], radius=True, delta_err=derr, lse_err=f["b_lse"])
    for n in ("dq", "dk", "dv"):
        _log("   ", U.compare(n, g[n], b[n], allow=b["r_" + n] + b["b_" + n], norm_rel=U.NORM_TOL, flip=b["r_" + n]))
    pk = _timed_instances_and_dkdv_probes(shape, ops, g["lse"], g["delta"], g)
    _assert_zero_rowsums(g, "dQ kernel")
    _assert_zero_rowsums(pk, "dK/dV kernel")
    # the row sums after the E5M2 cast along keys (the third probe)
    api = _api()
    pc = api.attn_bwd_dq(shape, ops, g["lse"], g["delta"], probe_cast=True)
    torch.cuda.synchronize()
    assert torch.equal(pc["dq"], g["dq"]) and torch.equal(pc["rowsum"], g["rowsum"])
    U.compare("rowsum_cast", pc["rowsum_cast"], b["rowsum_cast"],
              allow=b["r_rowsum_cast"] + b["b_rowsum_cast"] + 1e-30, rel=0.0)


GROUP_SCALE_CASES = {
    # multi-query attention (one KV head for 8 query heads: the dK/dV head loop at its longest) with a
    # softmax scale other than 1/sqrt(d); the same at head dim 256; MLA dims, non-causal, small scale
    "mqa_d128_s0.25": (W.small("mqa128", batch=1, heads_q=8, heads_kv=1, seqlen=192, d_qk=128, d_v=128,
                                causal=True, kind="rmsnorm", seed=21), 0.25),
    "mqa_d256": (W.small("mqa256", batch=1, heads_q=4, heads_kv=1, seqlen=160, d_qk=256, d_v=256, causal=True,
                         kind="rmsnorm", seed=22), None),
    "mla_nc_s0.05": (W.small("mla_nc", batch=2, heads_q=2, heads_kv=2, seqlen=130, d_qk=192, d_v=128,
                             causal=False, kind="scaled", seed=23), 0.05),
}


@pytest.mark.parametrize("name", list(GROUP_SCALE_CASES))
def test_chain_query_groups_and_softmax_scale(name):
    """The matched chain with a large query group and an explicit softmax scale, against the oracle."""
    w, scale = GROUP_SCALE_CASES[name]
    api = _api()
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal, scale)
    shp = U.oracle_shape(w, shape.sigma)
    inputs = W.generate(w)
    _log(f"[chain groups/scale] {name} sigma={shape.sigma}")
    ref = U.run_oracle(inputs, shp, modes=("matched",))
    _, ops = _gpu_ops(inputs)
    g = api.fwd_delta_bwd(shape, ops, "matched", probe=True)
    torch.cuda.synchronize()
    f, r = ref["fwd"], ref["matched"]
    U.compare("O", g["o"], f["o"], allow=f["r_o"] + f["b_o"], norm_rel=U.NORM_TOL, flip=f["r_o"])
    U.compare("LSE", g["lse"], f["lse"], allow=f["b_lse"], rel=0.0)
    derr = A.delta_bound(ref["ops"], shp, "matched", lse=f["lse"], lse_err=f["b_lse"])
    U.compare("delta", g["delta"], r["delta"], allow=derr, rel=0.0)
    b = A.backward(ref["ops"], shp, f["lse"], r["delta"], radius=True, delta_err=derr, lse_err=f["b_lse"])
    for n in ("dq", "dk", "dv"):
        _log("   ", U.compare(n, g[n], b[n], allow=b["r_" + n] + b["b_" + n], norm_rel=U.NORM_TOL, flip=b["r_" + n]))
    pk = _timed_instances_and_dkdv_probes(shape, ops, g["lse"], g["delta"], g)
    _assert_zero_rowsums(g, "dQ kernel")
    _assert_zero_rowsums(pk, "dK/dV kernel")


# shapes for the head-split dK/dV entry, with the split each takes: the query heads of a KV
# group dealt to hs workgroups per key tile (1: no split, no workspace)
HEAD_SPLIT_CASES = {
    "gqa_ragged": 2, "gqa_gain": 4, "mqa_d128_s0.25": 8, "tiny": 1, "mla": 1, "d256": 1, "gqa_nc": 4,
}
# non-causal, ragged: every key tile walks every query step, the last key tile is partly padding
SPLIT_ONLY = {
    "gqa_nc": W.small("gqa_nc", batch=1, heads_q=8, heads_kv=2, seqlen=250, d_qk=128, d_v=128, causal=False,
                      kind="rmsnorm", seed=24),
}


def _split_case(name):
    if name in SPLIT_ONLY:
        w = SPLIT_ONLY[name]
        api = _api()
        shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal)
        shp = U.oracle_shape(w, shape.sigma)
        inputs = W.generate(w)
        _log(f"[oracle] {name}")
        return w, inputs, shape, shp, U.run_oracle(inputs, shp, modes=("matched",))
    if name in GROUP_SCALE_CASES:
        w, scale = GROUP_SCALE_CASES[name]
        api = _api()
        shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal, scale)
        shp = U.oracle_shape(w, shape.sigma)
        inputs = W.generate(w)
        _log(f"[oracle] {name}")
        return w, inputs, shape, shp, U.run_oracle(inputs, shp, modes=("matched",))
    return _case(name)


@pytest.mark.parametrize("name", list(HEAD_SPLIT_CASES))
def test_head_split_dkdv_parity(name):
    """dm_attn_bwd_dkdv_ws: dK, dV against the oracle (matched delta) with the split's partial sums
    in a workspace that holds garbage on entry; bit-identical on a second call; identical to
    dm_attn_bwd_dkdv where the shape takes no split."""
    w, inputs, shape, shp, ref = _split_case(name)
    api = _api()
    hs = HEAD_SPLIT_CASES[name]
    need = api.dkdv_workspace_size(shape)
    assert need == (0 if hs == 1 else hs * w.batch * w.heads_kv * w.seqlen * 2 * w.d_qk * 4), need
    _log(f"[head split] {name}: {need} bytes of workspace")
    _, ops = _gpu_ops(inputs)
    r = ref["matched"]
    lse32, d32 = _f32(ref["fwd"]["lse"]), _f32(r["delta"])
    ws = torch.full((max(need, 16) + 256,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes
    g1 = api.attn_bwd_dkdv_ws(shape, ops, lse32, d32, workspace=ws)
    g2 = api.attn_bwd_dkdv_ws(shape, ops, lse32, d32, workspace=ws[:max(need, 16)])
    plain = api.attn_bwd_dkdv(shape, ops, lse32, d32)
    torch.cuda.synchronize()
    b = r["bwd"]
    for n in ("dk", "dv"):
        _log("   ", U.compare(n, g1[n], b[n], allow=b["r_" + n] + b["b_" + n], norm_rel=U.NORM_TOL,
                              flip=b["r_" + n]))
        assert torch.equal(g1[n], g2[n]), n + ": head-split result differs between two calls"
        if hs == 1:
            assert torch.equal(g1[n], plain[n]), n + ": without a split the result must be dm_attn_bwd_dkdv's"


def test_head_split_workspace_errors():
    api = _api()
    w, inputs, shape, shp, ref = _case("gqa_gain")
    _, ops = _gpu_ops(inputs)
    lse32, d32 = _f32(ref["fwd"]["lse"]), _f32(ref["matched"]["delta"])
    need = api.dkdv_workspace_size(shape)
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(api.DmError, match="DM_ERR_WORKSPACE"):
        api.attn_bwd_dkdv_ws(shape, ops, lse32, d32, workspace=ws)
    ws = torch.empty(need + 32, dtype=torch.uint8, device="cuda")
    with pytest.raises(api.DmError, match="DM_ERR_ALIGN"):
        api.attn_bwd_dkdv_ws(shape, ops, lse32, d32, workspace=ws[8:])


@pytest.mark.parametrize("mode", ["stale", "do_matched"])
@pytest.mark.parametrize("name", ["gqa_ragged", "mla", "d256"])
def test_chain_saved_output_modes(name, mode):
    """Chain with delta from the kernel's own O: the oracle bound carries O's deviation into delta."""
    w, inputs, shape, shp, ref = _case(name)
    _log(f"[chain {mode}] {name}")
    api = _api()
    dev, ops = _gpu_ops(inputs)
    g = api.fwd_delta_bwd(shape, ops, mode, do=dev["do"])
    torch.cuda.synchronize()
    f = ref["fwd"]
    o_err = U.REL_TOL * float(np.sqrt(np.mean(f["o"] ** 2))) + f["r_o"] + f["b_o"]
    derr = A.delta_bound(ref["ops"], shp, mode, o=f["o"], do=ref["do"], o_err=o_err)
    U.compare("delta", g["delta"], ref[mode]["delta"], allow=derr, rel=0.0)
    b = A.backward(ref["ops"], shp, f["lse"], ref[mode]["delta"], radius=True, delta_err=derr, lse_err=f["b_lse"])
    for n in ("dq", "dk", "dv"):
        U.compare(n, g[n], b[n], allow=b["r_" + n] + b["b_" + n])


# ---------------------------------------------------------------------------
# metamorphic and determinism checks (GPU only)
# ---------------------------------------------------------------------------

def test_power_of_two_scaling_is_exact():
    w = SMALL["gqa_ragged"]
    inputs = W.generate(w)
    api = _api()
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal)
    _, ops = _gpu_ops(inputs)
    scaled = dict(inputs, v=(inputs["v"].float() * 2).bfloat16(), do=(inputs["do"].float() * 4).bfloat16())
    _, ops2 = _gpu_ops(scaled)
    g1 = api.fwd_delta_bwd(shape, ops, "matched")
    g2 = api.fwd_delta_bwd(shape, ops2, "matched")
    torch.cuda.synchronize()
    assert torch.equal(g1["o"] * 2, g2["o"]) and torch.equal(g1["lse"], g2["lse"])
    assert torch.equal(g1["delta"] * 8, g2["delta"])
    assert torch.equal(g1["dk"] * 8, g2["dk"]) and torch.equal(g1["dv"] * 4, g2["dv"])
    assert torch.equal(g1["dq"] * 8, g2["dq"])


def test_run_to_run_determinism():
    w = SMALL["gqa_gain"]
    inputs = W.generate(w)
    api = _api()
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal)
    _, ops = _gpu_ops(inputs)
    a = api.fwd_delta_bwd(shape, ops, "matched")
    b = api.fwd_delta_bwd(shape, ops, "matched")
    torch.cuda.synchronize()
    for n in ("o", "lse", "delta", "dk", "dv", "dq"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("name", ["gqa_ragged", "mla", "d256"])
def test_split_backward_matches_fused(name):
    """dm_attn_bwd_dkdv + dm_attn_bwd_dq (here on two streams) give dm_attn_bwd's bits."""
    w = SMALL[name]
    inputs = W.generate(w)
    api = _api()
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal)
    _, ops = _gpu_ops(inputs)
    f = api.fwd_delta_bwd(shape, ops, "matched", probe=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    a = api.attn_bwd_dkdv(shape, ops, f["lse"], f["delta"])
    with torch.cuda.stream(side):
        q = api.attn_bwd_dq(shape, ops, f["lse"], f["delta"], probe=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for n in ("dk", "dv"):
        assert torch.equal(a[n], f[n]), n
    for n in ("dq", "rowsum", "rowabs"):
        assert torch.equal(q[n], f[n]), n


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128), (256, 256)], ids=lambda d: f"d{d[0]}x{d[1]}")
@pytest.mark.parametrize("L", [1, 33, 128, 129])
def test_short_and_ragged_lengths(L, dims):
    w = W.small("short", batch=1, heads_q=2, heads_kv=1, seqlen=L, d_qk=dims[0], d_v=dims[1], causal=True,
                kind="iid", seed=30 + L + dims[0])
    inputs = W.generate(w)
    api = _api()
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, L, w.d_qk, w.d_v, True)
    shp = U.oracle_shape(w, shape.sigma)
    ref = U.run_oracle(inputs, shp, modes=("matched",))
    _, ops = _gpu_ops(inputs)
    g = api.fwd_delta_bwd(shape, ops, "matched", probe=True)
    torch.cuda.synchronize()
    f = ref["fwd"]
    U.compare("O", g["o"], f["o"], allow=f["r_o"] + f["b_o"], norm_rel=U.NORM_TOL, flip=f["r_o"])
    derr = A.delta_bound(ref["ops"], shp, "matched", lse=f["lse"], lse_err=f["b_lse"])
    b = A.backward(ref["ops"], shp, f["lse"], ref["matched"]["delta"], radius=True, delta_err=derr,
                   lse_err=f["b_lse"])
    for n in ("dq", "dk", "dv"):
        U.compare(n, g[n], b[n], allow=b["r_" + n] + b["b_" + n], norm_rel=U.NORM_TOL, flip=b["r_" + n])
    pk = _timed_instances_and_dkdv_probes(shape, ops, g["lse"], g["delta"], g)
    _assert_zero_rowsums(g, "dQ kernel")
    _assert_zero_rowsums(pk, "dK/dV kernel")
    # causal row 0 sees only key 0: O_0 is the decoded V row (P^' = 1 exactly; P' and l are 1 to
    # within the FP32 rounding of exp2(fma(s, c2, -round(mu c2))), a few ulp)
    v0 = ref["ops"]["v_s"][0, 0, 0]
    np.testing.assert_allclose(U.to64(g["o"])[0, 0, 0], v0, rtol=2.0 ** -21, atol=0)


def test_zero_length_is_a_noop():
    api = _api()
    shape = api.AttnShape(1, 1, 1, 0, 64, 64, True)
    z = torch.zeros(16, dtype=torch.uint8, device="cuda")
    s = torch.zeros(4, dtype=torch.float32, device="cuda")
    op = api.Fp8Operand(z, s)
    o = torch.full((4,), 7.0, device="cuda")
    api.attn_fwd(shape, op, op, op, o=o, lse=o)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)


def test_zero_inputs_and_zero_queries():
    """All-zero operands (clamped scales) and Q = 0 (uniform attention: O is a running mean of V_hat)."""
    w = W.small("zeros", batch=1, heads_q=1, heads_kv=1, seqlen=200, d_qk=128, d_v=128, causal=True,
                kind="iid", seed=40)
    inputs = W.generate(w)
    inputs["q"] = torch.zeros_like(inputs["q"])
    api = _api()
    shape = api.AttnShape(1, 1, 1, 200, 128, 128, True)
    _, ops = _gpu_ops(inputs)
    g = api.fwd_delta_bwd(shape, ops, "matched", probe=True)
    torch.cuda.synchronize()
    _timed_instances_and_dkdv_probes(shape, ops, g["lse"], g["delta"], g)
    vs = A.decode_operands({"v_s": A.quantize_sequence(U.to64(inputs["v"]), "e4m3")}, 200)["v_s"][0, 0]
    n = np.arange(1, 201)[:, None]
    mean = np.cumsum(vs, axis=0) / n
    # every probability is exactly 1 before normalising: only the P V product's accumulation error remains
    U.compare("O", g["o"][0, 0], mean, rel=1e-6, allow=A.GAMMA * np.cumsum(np.abs(vs), axis=0) / n)
    assert np.allclose(U.to64(g["lse"])[0, 0], np.log(np.arange(1, 201)), atol=1e-5)
    zero = {n: torch.zeros_like(t) for n, t in inputs.items()}
    _, zops = _gpu_ops(zero)
    gz = api.fwd_delta_bwd(shape, zops, "matched", probe=True)
    torch.cuda.synchronize()
    pz = _timed_instances_and_dkdv_probes(shape, zops, gz["lse"], gz["delta"], gz)
    for n in ("o", "delta", "dq", "dk", "dv"):
        assert torch.count_nonzero(gz[n]) == 0, n
    for n in ("rowsum", "rowabs"):
        assert torch.count_nonzero(gz[n]) == 0 and torch.count_nonzero(pz[n]) == 0, n
