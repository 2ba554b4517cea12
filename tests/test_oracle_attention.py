"""Pins of the oracle's attention forward, row correction and backward (CPU only).

Pinned against: torch's float64 scaled-dot-product attention and its autograd
(identity codec), central finite differences, the exact identities of the
Delta-Matching project page (zero row sums, the residual split, the centered
correction), closed forms (causal row 0, zero queries), a brute-force
streaming loop for the chunked running maximum, GQA by explicit repetition,
and power-of-two metamorphic scaling.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8


def _rand_ops(rng, B, Hq, Hkv, L, dqk, dv, quant=True, q=None, k=None, v=None, do=None):
    q = rng.standard_normal((B, Hq, L, dqk)) if q is None else q
    k = rng.standard_normal((B, Hkv, L, dqk)) if k is None else k
    v = rng.standard_normal((B, Hkv, L, dv)) if v is None else v
    do = 0.1 * rng.standard_normal((B, Hq, L, dv)) if do is None else do
    if quant:
        ops = A.decode_operands(A.quantize_operands(q, k, v, do), L)
    else:
        ops = {"q_c": q, "q_s": q, "k_c": k, "k_s": k, "v_c": v, "v_s": v, "do_c": do, "do_s": do}
    return q, k, v, do, ops


def _shape(B, Hq, Hkv, L, dqk, dv, causal):
    return A.Shape(B, Hq, Hkv, L, dqk, dv, causal, 1.0 / np.sqrt(dqk))


def _torch_attn(q, k, v, do, causal, G):
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    kk = kt.repeat_interleave(G, dim=1)
    vv = vt.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kk, vv, is_causal=causal)
    (o * torch.tensor(do)).sum().backward()
    lse = torch.logsumexp(
        (qt @ kk.transpose(-1, -2) / np.sqrt(q.shape[-1])).masked_fill(
            torch.ones(q.shape[2], q.shape[2], dtype=torch.bool).triu(1) if causal
            else torch.zeros(q.shape[2], q.shape[2], dtype=torch.bool), float("-inf")), dim=-1)
    return (o.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", [(2, 1, 64, 64), (4, 2, 48, 32), (2, 2, 96, 64)])
def test_identity_codec_matches_torch_sdpa_and_autograd(causal, dims):
    Hq, Hkv, dqk, dv = dims
    rng = np.random.default_rng(1)
    B, L = 2, 200
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, dqk, dv, quant=False)
    shp = _shape(B, Hq, Hkv, L, dqk, dv, causal)
    f = A.forward(ops, shp, cast=False)
    o, lse, dq, dk, dv_ = _torch_attn(q, k, v, do, causal, Hq // Hkv)
    assert np.abs(f["o"] - o).max() < 1e-12
    assert np.abs(f["lse"] - lse).max() < 1e-12
    for mode in A.MODES:   # without quantization the three corrections coincide
        d = A.delta(ops, shp, mode, o=f["o"], do=do, lse=f["lse"])
        b = A.backward(ops, shp, f["lse"], d, cast=False)
        assert np.abs(b["dq"] - dq).max() < 1e-11
        assert np.abs(b["dk"] - dk).max() < 1e-11
        assert np.abs(b["dv"] - dv_).max() < 1e-11


def test_finite_differences_tiny():
    """Central differences of sum(O * dO) match dQ, dK, dV (identity codec)."""
    rng = np.random.default_rng(2)
    B, Hq, Hkv, L, d = 1, 2, 1, 40, 8
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d, quant=False)
    shp = _shape(B, Hq, Hkv, L, d, d, True)

    def loss(qq, kk, vv):
        o = {"q_c": qq, "k_c": kk, "v_s": vv}
        return float((A.forward(o, shp, cast=False)["o"] * do).sum())

    f = A.forward(ops, shp, cast=False)
    dlt = A.delta(ops, shp, "matched", lse=f["lse"])
    g = A.backward(ops, shp, f["lse"], dlt, cast=False)
    h = 1e-5
    for name, grad, idx in (("q", g["dq"], [(0, 1, 7, 3), (0, 0, 39, 0)]),
                            ("k", g["dk"], [(0, 0, 3, 5), (0, 0, 0, 1)]),
                            ("v", g["dv"], [(0, 0, 11, 2), (0, 0, 39, 7)])):
        for ix in idx:
            arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            arrs[name][ix] += h
            lp = loss(arrs["q"], arrs["k"], arrs["v"])
            arrs[name][ix] -= 2 * h
            lm = loss(arrs["q"], arrs["k"], arrs["v"])
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[ix]) <= 1e-6 * max(1.0, abs(fd)), (name, ix, fd, grad[ix])


def test_a_matched_delta_equals_saved_output_shortcut_without_quantization():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, L, d = 1, 2, 2, 160, 32
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d, quant=False)
    shp = _shape(B, Hq, Hkv, L, d, d, True)
    f = A.forward(ops, shp, cast=False)
    dm = A.delta(ops, shp, "matched", lse=f["lse"])
    ds = A.delta(ops, shp, "stale", o=f["o"], do=do)
    assert np.abs(dm - ds).max() <= 1e-12 * np.abs(ds).max()


@pytest.mark.parametrize("causal", [False, True])
def test_b_matched_rows_sum_to_zero(causal):
    rng = np.random.default_rng(4)
    B, Hq, Hkv, L, d = 1, 2, 1, 300, 64
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d)
    shp = _shape(B, Hq, Hkv, L, d, d, causal)
    f = A.forward(ops, shp)
    dm = A.delta(ops, shp, "matched", lse=f["lse"])
    b = A.backward(ops, shp, f["lse"], dm)
    assert np.all(np.abs(b["rowsum"]) <= 1e-12 * b["rowabs"])
    # the stale correction does not have this property under quantization
    ds = A.delta(ops, shp, "stale", o=f["o"], do=do)
    bs = A.backward(ops, shp, f["lse"], ds)
    assert np.median(np.abs(bs["rowsum"]) / bs["rowabs"]) > 1e-4


def _terms(ops, q, k, v, do, shp, shared_v):
    """T_P, T_dO, T_V of the residual split for head (0, 0)."""
    Q, K, Vs, Vc, dOc = ops["q_c"][0, 0], ops["k_c"][0, 0], ops["v_s"][0, 0], ops["v_c"][0, 0], ops["do_c"][0, 0]
    if shared_v:
        Vc = Vs
    L = shp.seqlen
    f = A.forward_rows(Q, K, Vs, shp.sigma, shp.causal, 0, L)
    P = A.probs_rows(Q, K, f["lse"], shp.sigma, shp.causal, 0, L)
    O = f["o"]
    TP = np.einsum("ik,ik->i", dOc, P @ Vs - O)            # <dO_hat, (P - P_hat) V_hat>
    TdO = np.einsum("ik,ik->i", dOc - do[0, 0], O)          # <dO_hat - dO, P_hat V_hat>
    TV = np.einsum("ik,ik->i", dOc, P @ (Vc - Vs))          # V blocked differently in the two products
    return f, P, TP, TdO, TV


@pytest.mark.parametrize("shared_v", [True, False])
def test_c_residual_split(shared_v):
    """Stale residual = probability term + dO term (+ V term when V is blocked twice)."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, L, d = 1, 1, 1, 256, 64
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d)
    if shared_v:
        ops = dict(ops, v_c=ops["v_s"])
    shp = _shape(B, Hq, Hkv, L, d, d, True)
    f, P, TP, TdO, TV = _terms(ops, q, k, v, do, shp, shared_v)
    fo = A.forward(ops, shp)
    ds = A.delta(ops, shp, "stale", o=fo["o"], do=do)
    dd = A.delta(ops, shp, "do_matched", o=fo["o"], do=do)
    rs = A.backward(ops, shp, fo["lse"], ds)["rowsum"][0, 0]
    rd = A.backward(ops, shp, fo["lse"], dd)["rowsum"][0, 0]
    scale = np.abs(TP).max() + np.abs(TdO).max()
    assert np.abs(rs - (TP + TdO + TV)).max() <= 1e-12 * scale
    assert np.abs(rd - (TP + TV)).max() <= 1e-12 * scale
    if shared_v:
        assert np.all(TV == 0)
    assert np.abs(TP).max() > 1e-3 * scale and np.abs(TdO).max() > 1e-3 * scale


def test_d_stale_equals_centered_plus_eps_p():
    """dS_stale - dS_matched = eps_i P_ij, seen through dQ (no gradient cast) and the row sums."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, L, d = 1, 2, 1, 192, 32
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d)
    shp = _shape(B, Hq, Hkv, L, d, d, True)
    f = A.forward(ops, shp)
    dm = A.delta(ops, shp, "matched", lse=f["lse"])
    ds = A.delta(ops, shp, "stale", o=f["o"], do=do)
    bm = A.backward(ops, shp, f["lse"], dm, cast=False)
    bs = A.backward(ops, shp, f["lse"], ds, cast=False)
    eps = dm - ds
    for h in range(Hq):
        P = A.probs_rows(ops["q_c"][0, h], ops["k_c"][0, 0], f["lse"][0, h], shp.sigma, True, 0, L)
        want = shp.sigma * eps[0, h][:, None] * (P @ ops["k_s"][0, 0])
        got = bs["dq"][0, h] - bm["dq"][0, h]
        assert np.abs(got - want).max() <= 1e-12 * np.abs(bm["dq"]).max()
    assert np.abs((bs["rowsum"] - bm["rowsum"]) - eps).max() <= 1e-12 * np.abs(eps).max()


def test_closed_forms():
    rng = np.random.default_rng(8)
    B, H, L, d = 1, 1, 300, 64
    # causal row 0 sees one key: O_0 = V_hat<s>[0] exactly
    q, k, v, do, ops = _rand_ops(rng, B, H, H, L, d, d)
    shp = _shape(B, H, H, L, d, d, True)
    f = A.forward(ops, shp)
    assert np.array_equal(f["o"][0, 0, 0], ops["v_s"][0, 0, 0])
    # zero queries: every unmasked probability is 1 before normalising, so O_i is a plain mean
    q0 = np.zeros_like(q)
    _, _, _, _, ops0 = _rand_ops(rng, B, H, H, L, d, d, q=q0, k=k, v=v, do=do)
    f0 = A.forward(ops0, shp)
    cm = np.cumsum(ops0["v_s"][0, 0], axis=0) / np.arange(1, L + 1)[:, None]
    assert np.abs(f0["o"][0, 0] - cm).max() <= 1e-13
    assert np.allclose(f0["lse"][0, 0], np.log(np.arange(1, L + 1)), atol=1e-13, rtol=0)


def test_running_max_chunks_brute_force_stream():
    """A literal streaming loop (row by row, 128-key chunk by chunk) reproduces forward()."""
    rng = np.random.default_rng(9)
    L, d = 300, 16
    Q = rng.standard_normal((L, d)) * 2
    K = rng.standard_normal((L, d)) * 2
    V = rng.standard_normal((L, d))
    sig = 0.25
    for causal in (False, True):
        ref = A.forward_rows(Q, K, V, sig, causal, 0, L)
        for i in (0, 1, 127, 128, 200, 299):
            mu = -np.inf
            acc = np.zeros(d)
            l = 0.0
            for c0 in range(0, 384, 128):
                s = np.full(128, -np.inf)
                for jj in range(128):
                    j = c0 + jj
                    if j < L and (not causal or j <= i):
                        s[jj] = sig * float(Q[i] @ K[j])
                new_mu = max(mu, s.max())
                if new_mu == -np.inf:
                    continue
                alpha = 0.0 if mu == -np.inf else np.exp(mu - new_mu)
                p = np.exp(s - new_mu)
                _, _, ph = fp8.quantize_lastaxis(p[None, :], "e4m3")
                vv = np.zeros((128, d))
                n = max(0, min(L - c0, 128))
                vv[:n] = V[c0:c0 + n]
                acc = acc * alpha + ph[0] @ vv
                l = l * alpha + p.sum()
                mu = new_mu
            assert np.abs(acc / l - ref["o"][i]).max() < 1e-12
            assert abs(mu + np.log(l) - ref["lse"][i]) < 1e-12


def test_gqa_equals_explicit_repeat():
    rng = np.random.default_rng(10)
    B, Hq, Hkv, L, d = 1, 4, 2, 160, 32
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d)
    shp = _shape(B, Hq, Hkv, L, d, d, True)
    rep = {n: (np.repeat(a, 2, axis=1) if n[0] in "kv" else a) for n, a in ops.items()}
    shp_r = _shape(B, Hq, Hq, L, d, d, True)
    f, fr = A.forward(ops, shp), A.forward(rep, shp_r)
    assert np.array_equal(f["o"], fr["o"]) and np.array_equal(f["lse"], fr["lse"])
    dm = A.delta(ops, shp, "matched", lse=f["lse"])
    b, br = A.backward(ops, shp, f["lse"], dm), A.backward(rep, shp_r, f["lse"], dm)
    assert np.abs(b["dq"] - br["dq"]).max() == 0
    assert np.abs(b["dk"] - br["dk"].reshape(B, Hkv, 2, L, d).sum(2)).max() < 1e-12
    assert np.abs(b["dv"] - br["dv"].reshape(B, Hkv, 2, L, d).sum(2)).max() < 1e-12


def test_power_of_two_metamorphic():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, L, d = 1, 2, 1, 224, 64
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d)
    _, _, _, _, ops2 = _rand_ops(rng, B, Hq, Hkv, L, d, d, q=q, k=k, v=2 * v, do=4 * do)
    shp = _shape(B, Hq, Hkv, L, d, d, True)
    f, f2 = A.forward(ops, shp), A.forward(ops2, shp)
    assert np.array_equal(2 * f["o"], f2["o"]) and np.array_equal(f["lse"], f2["lse"])
    dm, dm2 = A.delta(ops, shp, "matched", lse=f["lse"]), A.delta(ops2, shp, "matched", lse=f2["lse"])
    assert np.allclose(8 * dm, dm2, rtol=1e-14, atol=0)
    b, b2 = A.backward(ops, shp, f["lse"], dm), A.backward(ops2, shp, f2["lse"], 8 * dm)
    assert np.array_equal(8 * b["dq"], b2["dq"]) and np.array_equal(8 * b["dk"], b2["dk"])
    assert np.array_equal(4 * b["dv"], b2["dv"])


def test_radius_covers_small_perturbations():
    """Perturbing the operands within the kernel's error budget moves results only within the bound.

    The perturbation (relative 2^-14 on the score operand, so |dS| <= 2^-14 A
    which is inside GAMMA * A; 1e-7 on LSE and delta) flips some ambiguous
    casts; the total change must stay inside radius + accumulation bound, and
    the flips must need the radius (without it the check fails).
    """
    rng = np.random.default_rng(13)
    B, Hq, Hkv, L, d = 1, 2, 1, 256, 64
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d)
    shp = _shape(B, Hq, Hkv, L, d, d, True)
    f = A.forward(ops, shp, radius=True)
    f_nc = A.forward(ops, shp, cast=False)
    dm = A.delta(ops, shp, "matched", lse=f["lse"])
    b = A.backward(ops, shp, f["lse"], dm, radius=True)
    b_nc = A.backward(ops, shp, f["lse"], dm, cast=False)
    assert f["n_flag"] > 0 and b["n_flag"] > 0
    needed = 0
    for t in range(3):
        pert = dict(ops)
        pert["q_c"] = ops["q_c"] * (1 + 2.0 ** -14 * rng.uniform(-1, 1, ops["q_c"].shape))
        fp, fp_nc = A.forward(pert, shp), A.forward(pert, shp, cast=False)
        diff = np.abs(fp["o"] - f["o"])
        assert np.all(diff <= f["r_o"] + f["b_o"])
        smooth = 3 * np.abs(fp_nc["o"] - f_nc["o"]).max()
        needed += int(np.any(diff > smooth + f["b_o"]))
        lse_p = f["lse"] * (1 + 1e-7 * rng.uniform(-1, 1, f["lse"].shape))
        dm_p = dm * (1 + 1e-7 * rng.uniform(-1, 1, dm.shape))
        bp, bp_nc = A.backward(pert, shp, lse_p, dm_p), A.backward(pert, shp, lse_p, dm_p, cast=False)
        for n in ("dq", "dk", "dv"):
            diff = np.abs(bp[n] - b[n])
            smooth = 3 * np.abs(bp_nc[n] - b_nc[n]).max()
            assert np.all(diff <= b["r_" + n] + b["b_" + n] + smooth), n
            needed += int(np.any(diff > smooth + b["b_" + n]))
    assert needed > 0


def test_row_subsets_match_full():
    rng = np.random.default_rng(14)
    B, Hq, Hkv, L, d = 1, 2, 1, 330, 64
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d)
    shp = _shape(B, Hq, Hkv, L, d, d, True)
    f = A.forward(ops, shp)
    dm = A.delta(ops, shp, "matched", lse=f["lse"])
    b = A.backward(ops, shp, f["lse"], dm)
    rows = [(32, 96), (256, L)]
    fs = A.forward(ops, shp, rows=rows)
    m = A._row_mask(L, rows)
    assert np.array_equal(fs["o"][:, :, m], f["o"][:, :, m]) and np.isnan(fs["o"][:, :, ~m]).all()
    bs = A.backward(ops, shp, f["lse"], dm, rows=rows)
    assert np.abs(bs["dq"][:, :, m] - b["dq"][:, :, m]).max() == 0
    assert np.abs(bs["dk"][:, :, 256:] - b["dk"][:, :, 256:]).max() < 1e-12
    assert np.abs(bs["dv"][:, :, 256:] - b["dv"][:, :, 256:]).max() < 1e-12


def test_quantized_layouts_brute_force():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((1, 2, 70, 64))
    c, s = A.quantize_channels(x, "e4m3")
    assert c.shape == (1, 2, 70, 64) and s.shape == (1, 2, 70, 2)
    for (h, r, blk) in ((0, 0, 0), (1, 69, 1)):
        cc, ss, _ = fp8.quantize_lastaxis(x[0, h, r, 32 * blk:32 * blk + 32][None], "e4m3")
        assert np.array_equal(c[0, h, r, 32 * blk:32 * blk + 32], cc[0]) and s[0, h, r, blk] == ss[0, 0]
    c, s = A.quantize_sequence(x, "e5m2")
    assert c.shape == (1, 2, 64, 96) and s.shape == (1, 2, 64, 3)
    col = np.zeros(96)
    col[:70] = x[0, 1, :, 5]
    cc, ss, _ = fp8.quantize_lastaxis(col[None], "e5m2")
    assert np.array_equal(c[0, 1, 5], cc[0]) and np.array_equal(s[0, 1, 5], ss[0])
    assert not c[0, :, :, 70:].any()
    back = A.dequantize_sequence(c, s, "e5m2", 70)
    assert back.shape == x.shape and np.abs(back - x).max() < 0.2 * np.abs(x).max()


@pytest.mark.parametrize("causal", [False, True])
def test_postcast_rowsum_is_the_sum_of_the_e5m2_cast(causal):
    """rowsum_cast is sum_j of dS cast to E5M2 in 32-key blocks: recomputed here from the
    oracle's pre-cast dS through torch's float8_e5m2 cast, with each block's scale taken
    from its definition (smallest power of two 2^k with amax <= 57344 * 2^k)."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, L, d = 1, 1, 1, 200, 64
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d)
    shp = _shape(B, Hq, Hkv, L, d, d, causal)
    f = A.forward(ops, shp)
    dm = A.delta(ops, shp, "matched", lse=f["lse"])
    oh = {n: ops[n][0, 0] for n in ("q_c", "k_c", "v_c", "do_c", "q_s", "k_s", "do_s")}
    r = A.backward_rows(oh, f["lse"][0, 0], dm[0, 0], shp.sigma, causal, 0, L, keep_ds=True)
    ds = np.zeros((L, 224))
    ds[:, :L] = r["ds"]
    blocks = ds.reshape(L, 7, 32)
    amax = np.abs(blocks).max(axis=-1)
    kexp = np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-300) / 57344.0)), -126).clip(-126, 127)
    # ceil(log2(.)) can land one above the minimum when the ratio is an exact power of two
    kexp = np.where((amax > 0) & (amax <= 57344.0 * np.exp2(kexp - 1)), kexp - 1, kexp)
    scale = np.exp2(kexp)[..., None]
    cast = torch.from_numpy(blocks / scale).to(torch.float8_e5m2).to(torch.float64).numpy() * scale
    want = cast.reshape(L, 224)[:, :L].sum(axis=1)
    assert np.allclose(r["rowsum_cast"], want, rtol=1e-12, atol=1e-300)
    # without the cast the post-cast sum is the pre-cast one; with matched delta that is ~0
    u = A.backward_rows(oh, f["lse"][0, 0], dm[0, 0], shp.sigma, causal, 0, L, cast=False)
    assert np.all(np.abs(u["rowsum_cast"] - u["rowsum"]) <= 1e-14 * u["rowabs"])
    assert np.all(np.abs(r["rowsum"]) <= 1e-12 * r["rowabs"])
    assert np.median(np.abs(r["rowsum_cast"]) / r["rowabs"]) > 1e-6   # the cast leaves a residual


def _torch_block_cast(x, fmax, dtype):
    """Cast x [..., 32 * nb] in blocks of 32 along the last axis through torch's float8 type, each
    block scaled by the smallest power of two 2^k (k in [-126, 127]) with amax <= fmax * 2^k."""
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    kexp = np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-300) / fmax)), -126).clip(-126, 127)
    kexp = np.where((amax > 0) & (amax <= fmax * np.exp2(kexp - 1)), kexp - 1, kexp)
    scale = np.exp2(kexp)[..., None]
    cast = torch.from_numpy(blocks / scale).to(dtype).to(torch.float64).numpy() * scale
    return cast.reshape(x.shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("L,r0", [(200, 0), (200, 96), (96, 0)])
def test_query_axis_casts_brute_force(causal, L, r0):
    """dV and dK use P and dS cast along the *query* axis: for every key column, 32-query blocks
    (a ragged last block zero-padded).  Recomputed here from independently formed P = exp(S - LSE)
    and the oracle's pre-cast dS through torch's float8_e4m3fn / float8_e5m2 casts (block scales
    from their definition): dV = P^<q>^T dO^<s>, dK = sigma dS^<q>^T Q^<s> over rows [r0, L).  A cast
    along keys instead, or a wrongly padded tail block, changes them (checked)."""
    rng = np.random.default_rng(40 + L + r0)
    B, Hq, Hkv, d = 1, 1, 1, 64
    # peaked rows (scores of several units): block maxima spread over many binades, so the
    # block scales differ between the two axes
    q = 3.0 * rng.standard_normal((B, Hq, L, d))
    q, k, v, do, ops = _rand_ops(rng, B, Hq, Hkv, L, d, d, q=q)
    shp = _shape(B, Hq, Hkv, L, d, d, causal)
    f = A.forward(ops, shp)
    dm = A.delta(ops, shp, "matched", lse=f["lse"])
    oh = {n: ops[n][0, 0] for n in ("q_c", "k_c", "v_c", "do_c", "q_s", "k_s", "do_s")}
    lse = f["lse"][0, 0, r0:L]
    r = A.backward_rows(oh, lse, dm[0, 0, r0:L], shp.sigma, causal, r0, L, keep_ds=True)
    # P from its definition, independently of the oracle's backward
    S = shp.sigma * (oh["q_c"][r0:L] @ oh["k_c"].T)
    if causal:
        S = np.where(np.arange(L)[None, :] > np.arange(r0, L)[:, None], -np.inf, S)
    P = np.exp(S - lse[:, None])
    n = L - r0
    n32 = (n + 31) // 32 * 32
    padP = np.zeros((n32, L))
    padP[:n] = P
    padS = np.zeros((n32, L))
    padS[:n] = r["ds"]
    # per key column: blocks of 32 consecutive queries (cast along axis 0 = transpose, last axis)
    Pq = _torch_block_cast(padP.T, 448.0, torch.float8_e4m3fn).T[:n]
    dSq = _torch_block_cast(padS.T, 57344.0, torch.float8_e5m2).T[:n]
    dv = Pq.T @ oh["do_s"][r0:L]
    dk = shp.sigma * (dSq.T @ oh["q_s"][r0:L])
    np.testing.assert_allclose(r["dv"], dv, rtol=1e-12, atol=1e-14 * np.abs(dv).max())
    np.testing.assert_allclose(r["dk"], dk, rtol=1e-12, atol=1e-14 * np.abs(dk).max())
    # the same casts along keys give different gradients (so the test tells the axes apart)
    Lk = (L + 31) // 32 * 32
    padK = np.zeros((n, Lk))
    padK[:, :L] = P
    Pk = _torch_block_cast(padK, 448.0, torch.float8_e4m3fn)[:, :L]
    assert np.abs(Pk.T @ oh["do_s"][r0:L] - r["dv"]).max() > 1e-6 * np.abs(dv).max()
    # and a tail block padded with anything but zeros (here 2, above every probability) changes
    # dV when the last block is ragged
    if n % 32:
        bad = padP.copy()
        bad[n:] = 2.0
        Pb = _torch_block_cast(bad.T, 448.0, torch.float8_e4m3fn).T[:n]
        assert not np.allclose(Pb.T @ oh["do_s"][r0:L], dv, rtol=1e-12, atol=0)
