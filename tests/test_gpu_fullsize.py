"""GPU parity at the full workload sizes, in the call sequence bench.py times.

The GPU runs the whole problem (quantize, forward, matched delta, dK/dV, dQ on
preallocated outputs, the same calls as bench.py).  The oracle checks the part
of it that it can compute exactly in about a minute: one batch entry and KV
group (the last of each, so the highest head and batch offsets are exercised),
and within it
  * FP8 codes and scales of every operand of the group: bit-exact;
  * at sequence lengths up to 8K: every query row, so O, LSE, delta and dQ are
    compared on all rows and dK, dV on all keys -- including the first key
    tiles, whose workgroups walk every query step of every head of the group;
  * at 64K: O, LSE, delta and dQ on sampled 32-row blocks and on the last 4096
    rows, and dK, dV on the last 4096 keys (under causal masking only rows at or
    after a key reach it, so those rows determine the keys completely).  The
    64K accumulation chains of the first key tiles (2048 chained instructions
    per dK/dV element) are covered by the instruction measurement in
    tests/test_gpu_mfma_accumulation.py, whose error does not grow with the
    chain.
The same elementwise and norm-wise bars as the small-size tests apply.  On every
row of the full problem, the matched-mode row sums |sum_j dS_ij| <= 1e-5
sum_j |P_ij dP_ij| are checked from the probes of both backward kernels (a
property that needs no oracle), and the probing instances are required to give
the timed instances' dQ, dK and dV bit for bit.

Where the shape's dK/dV grid is small enough for the head-split entry
(dm_attn_bwd_dkdv_ws, the call bench.py times) to split, the unsplit kernel's dK
and dV are compared as well.

The oracle runs in up to 16 spawned processes (one BLAS thread each): every
query head of the group split into row ranges; dK and dV are summed over the
ranges and heads.
"""
import concurrent.futures as cf
import multiprocessing
import sys
import time

import numpy as np
import pytest
import torch

from fp8_attention_amd import workloads as W
from oracle import attention as A
from tests import parity_util as U

pytestmark = pytest.mark.gpu

# workload -> rows the oracle covers: None (every row), or (tail, number of sampled 32-row
# blocks before the tail)
CASES = {
    "gqa_4k": None,
    "gqa_8k": None,
    "gqa_64k": (4096, 8),
    "mla_4k": None,
    "gqa_d256_4k": None,
    "gqa_8k_b1": None,
}
# the long-context head geometry at batch 1: its dK/dV grid (64 key tiles x 8 KV heads) is small
# enough for the head split (two workgroups per key tile), so the timed call splits at 8K
EXTRA_WORKLOADS = {
    "gqa_8k_b1": W.small("gqa_8k_b1", batch=1, heads_q=32, heads_kv=8, seqlen=8192, d_qk=128, d_v=128,
                         causal=True, kind="rmsnorm", q_gain7=2.0, k_gain7=5.4, seed=1006),
}
WORKERS = 16


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _rows(L: int, spec):
    """32-aligned row ranges the oracle covers, and the first row of the contiguous tail."""
    if spec is None:
        return [(0, L)], 0
    tail, nblocks = spec
    t0 = L - tail
    starts = sorted({int(s) // 32 * 32 for s in np.linspace(0, t0 - 32, nblocks)})
    return [(s, s + 32) for s in starts] + [(t0, L)], t0


def _split(ranges, parts):
    """Cut the row ranges into about ``parts`` pieces of similar size (32-aligned)."""
    total = sum(b - a for a, b in ranges)
    size = max(32, -(-total // parts) // 32 * 32)
    out, cur, n = [], [], 0
    for a, b in ranges:
        while a < b:
            take = min(b - a, size - n)
            cur.append((a, a + take))
            n += take
            a += take
            if n == size:
                out.append(cur)
                cur, n = [], 0
    if cur:
        out.append(cur)
    return out


def _oracle_part(q, k, v, do, shp, rows, key0, want_codes):
    """Oracle chain for one query head on some row ranges (run in a worker process).

    Returns the row-wise results on those rows only, dK/dV contributions of those rows
    to keys [key0, L), and (want_codes) the head's quantized operands."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        r = U.oracle_head_chain(q, k, v, do, shp, rows)
    idx = np.concatenate([np.arange(a, b) for a, b in rows])
    f, bw = r["fwd"], r["bwd"]
    out = {"idx": idx}
    for n in ("o", "r_o", "b_o"):
        out[n] = f[n][0, 0, idx]
    for n in ("lse", "b_lse"):
        out[n] = f[n][0, 0, idx]
    out["delta"], out["derr"] = r["delta"][0, 0, idx], r["derr"][0, 0, idx]
    for n in ("dq", "r_dq", "b_dq"):
        out[n] = bw[n][0, 0, idx]
    for n in ("dk", "dv", "r_dk", "b_dk", "r_dv", "b_dv"):
        out[n] = bw[n][0, 0, key0:]
    if want_codes:
        out["qops"] = r["qops"]
    return out


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", list(CASES))
def test_fullsize_chain_sampled(name):
    from fp8_attention_amd import api
    w = EXTRA_WORKLOADS[name] if name in EXTRA_WORKLOADS else W.WORKLOADS[name]
    B, Hq, Hkv, L, G = w.batch, w.heads_q, w.heads_kv, w.seqlen, w.group
    _log(f"[fullsize] {name}: {w}")
    inputs = W.generate(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    shape = api.AttnShape(B, Hq, Hkv, L, w.d_qk, w.d_v, w.causal)
    ops = api.quantize_operands(dev["q"], dev["k"], dev["v"], dev["do"])
    o = torch.empty((B, Hq, L, w.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq = torch.empty((B, Hq, L, w.d_qk), dtype=torch.float32, device="cuda")
    dk = torch.empty((B, Hkv, L, w.d_qk), dtype=torch.float32, device="cuda")
    dv = torch.empty((B, Hkv, L, w.d_v), dtype=torch.float32, device="cuda")
    # the timed step of bench.py
    api.attn_fwd(shape, ops["q_c"], ops["k_c"], ops["v_s"], o=o, lse=lse)
    api.attn_delta(shape, "matched", do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"], v_c=ops["v_c"],
                   lse=lse, out=delta)
    need = api.dkdv_workspace_size(shape)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    api.attn_bwd_dkdv_ws(shape, ops, lse, delta, workspace=ws, dk=dk, dv=dv)
    api.attn_bwd_dq(shape, ops, lse, delta, dq=dq)
    # the row-sum probes of both backward kernels over the whole problem; the probing
    # instances must reproduce the timed ones bit for bit
    pq = api.attn_bwd_dq(shape, ops, lse, delta, probe=True)
    pk = api.attn_bwd_dkdv(shape, ops, lse, delta, probe=True)
    # a small grid takes the head split in the timed step; then the unsplit kernel (whose
    # arithmetic the probing instance repeats) is checked as well
    unsplit = api.attn_bwd_dkdv(shape, ops, lse, delta) if need else {"dk": dk, "dv": dv}
    torch.cuda.synchronize()
    _log("   gpu done" + (f"; timed dK/dV with the head split ({need >> 20} MiB workspace)" if need else ""))
    assert torch.equal(pq["dq"], dq), "probing dQ instance differs from the timed one"
    assert torch.equal(pk["dk"], unsplit["dk"]) and torch.equal(pk["dv"], unsplit["dv"]), \
        "probing dK/dV instance differs from the unsplit timed one"
    for who, p in (("dQ kernel", pq), ("dK/dV kernel", pk)):
        rs, ra = U.to64(p["rowsum"]), U.to64(p["rowabs"])
        ratio = np.abs(rs) / np.maximum(ra, 1e-300)
        _log(f"   row sums ({who}): max |sum dS| / sum |P dP| = {float(ratio.max()):.2e}, "
             f"mean {float(ratio.mean()):.2e} over {rs.size} rows")
        assert np.all(np.abs(rs) <= U.ROWSUM_TOL * ra), f"{who}: row-sum ratio max {float(ratio.max()):.3e}"
    del pq, pk

    # oracle on the last batch entry and KV group
    b, g = B - 1, Hkv - 1
    sel = U.select_group(inputs, w, b, g)
    shp = A.Shape(1, 1, 1, L, w.d_qk, w.d_v, bool(w.causal), shape.sigma)
    rows, key0 = _rows(L, CASES[name])
    parts = _split(rows, max(1, WORKERS // G))
    t0 = time.perf_counter()
    k64, v64 = U.to64(sel["k"]), U.to64(sel["v"])
    qh = [U.to64(sel["q"][:, j:j + 1]) for j in range(G)]
    dh = [U.to64(sel["do"][:, j:j + 1]) for j in range(G)]
    ctx = multiprocessing.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=min(WORKERS, G * len(parts)), mp_context=ctx) as ex:
        futs = {ex.submit(_oracle_part, qh[j], k64, v64, dh[j], shp, part, key0, i == 0): (j, i)
                for j in range(G) for i, part in enumerate(parts)}
        res = {}
        pending = set(futs)
        while pending:
            done, pending = cf.wait(pending, timeout=30)
            for fu in done:
                res[futs[fu]] = fu.result()
            _log(f"   oracle: {len(res)} of {len(futs)} parts after {time.perf_counter() - t0:.0f} s")
    _log(f"   oracle {time.perf_counter() - t0:.1f} s on rows {rows} of {G} head(s), {len(parts)} part(s) each")

    idx = np.concatenate([np.arange(a, c) for a, c in rows])
    pos = {int(r): n for n, r in enumerate(idx)}
    nrow = len(idx)
    f = {n: np.full((1, G, nrow) + (() if n in ("lse", "b_lse") else (w.d_v,)), np.nan)
         for n in ("o", "r_o", "b_o", "lse", "b_lse")}
    d, derr = np.full((1, G, nrow), np.nan), np.full((1, G, nrow), np.nan)
    r = {n: np.full((1, G, nrow, w.d_qk), np.nan) for n in ("dq", "r_dq", "b_dq")}
    nk = L - key0
    for n in ("dk", "dv", "r_dk", "b_dk", "r_dv", "b_dv"):
        r[n] = np.zeros((1, 1, nk, w.d_qk if n.endswith("dk") else w.d_v))
    for (j, i), part in res.items():
        sl = np.array([pos[int(x)] for x in part["idx"]])
        for n in f:
            f[n][0, j, sl] = part[n]
        d[0, j, sl], derr[0, j, sl] = part["delta"], part["derr"]
        for n in ("dq", "r_dq", "b_dq"):
            r[n][0, j, sl] = part[n]
        for n in ("dk", "dv", "r_dk", "b_dk", "r_dv", "b_dv"):
            r[n][0, 0] += part[n]                              # summed over row ranges and the group's heads
    assert not np.isnan(d).any()

    hs = slice(g * G, (g + 1) * G)
    L32 = (L + 31) // 32 * 32
    for n in res[(0, 0)]["qops"]:
        if n[0] in "qd":                                       # q_*, do_*: per query head
            codes = np.concatenate([res[(j, 0)]["qops"][n][0] for j in range(G)], axis=1)
            scales = np.concatenate([res[(j, 0)]["qops"][n][1] for j in range(G)], axis=1)
            hsel = hs
        else:                                                  # k_*, v_*: the KV head
            codes, scales = res[(0, 0)]["qops"][n]
            hsel = slice(g, g + 1)
        gc = ops[n].codes[b:b + 1, hsel].cpu().numpy()
        gs = ops[n].scales[b:b + 1, hsel].cpu().numpy().astype(np.float64)
        if n.endswith("_c"):
            gc, gs = gc[..., :L, :], gs[..., :L, :]
        else:
            gc, gs = gc[..., :L32], gs[..., :L32 // 32]
        assert np.array_equal(gc, codes), n + " codes"
        assert np.array_equal(gs, scales), n + " scales"

    ti = torch.from_numpy(idx).cuda()
    pick = lambda t: t[b:b + 1, hs].index_select(2, ti)        # noqa: E731
    U.compare("O", pick(o), f["o"], allow=f["r_o"] + f["b_o"], norm_rel=U.NORM_TOL, flip=f["r_o"])
    U.compare("LSE", pick(lse), f["lse"], allow=f["b_lse"], rel=0.0)
    U.compare("delta", pick(delta), d, allow=derr, rel=0.0)
    _log("   ", U.compare("dq", pick(dq), r["dq"], allow=r["r_dq"] + r["b_dq"], norm_rel=U.NORM_TOL, flip=r["r_dq"]))
    outs = [("dk", "dk", dk), ("dv", "dv", dv)]
    if need:
        outs += [(n + " (unsplit)", n, unsplit[n]) for n in ("dk", "dv")]
    for label, n, full in outs:
        t = full[b:b + 1, g:g + 1, key0:]
        _log("   ", U.compare(label, t, r[n], allow=r["r_" + n] + r["b_" + n], norm_rel=U.NORM_TOL,
                              flip=r["r_" + n]))
        if key0 == 0:
            # the first key tile on its own: its workgroup walks every query step of every head
            first = slice(0, 128)
            _log("   ", U.compare(label + "[keys<128]", t[:, :, first], r[n][:, :, first],
                                  allow=(r["r_" + n] + r["b_" + n])[:, :, first], norm_rel=U.NORM_TOL,
                                  flip=r["r_" + n][:, :, first]))


@pytest.mark.parametrize("name", ["gqa_4k", "gqa_8k"])
def test_postcast_rowsum_residual_stale_vs_matched(name):
    """Direction of the project page's kernel probe (section 03): after dS is cast to FP8,
    the normalized row-sum residual |sum_j dS^<k>_ij| / sum_j |P_ij dP^_ij| is larger with
    the stale correction than with Delta-Matching (the page reports 5.3-6.3x on its
    models' activations; these synthetic inputs only fix the sign of the comparison).
    Both corrections start from the same GPU forward; the stale one from the bf16 dO."""
    from fp8_attention_amd import api
    w = W.WORKLOADS[name]
    inputs = W.generate(w)
    dev = {n: t.cuda() for n, t in inputs.items()}
    shape = api.AttnShape(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.d_qk, w.d_v, w.causal)
    ops = api.quantize_operands(dev["q"], dev["k"], dev["v"], dev["do"])
    o, lse = api.attn_fwd(shape, ops["q_c"], ops["k_c"], ops["v_s"])
    res = {}
    for mode in ("stale", "matched"):
        if mode == "stale":
            d = api.attn_delta(shape, mode, o=o, do=dev["do"])
        else:
            d = api.attn_delta(shape, mode, do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"], v_c=ops["v_c"],
                               lse=lse)
        p = api.attn_bwd_dq(shape, ops, lse, d, probe_cast=True)
        torch.cuda.synchronize()
        ra = U.to64(p["rowabs"])
        res[mode] = (np.abs(U.to64(p["rowsum"])) / ra, np.abs(U.to64(p["rowsum_cast"])) / ra)
    pre = np.mean(res["stale"][0]) / np.mean(res["matched"][0])
    post = np.mean(res["stale"][1]) / np.mean(res["matched"][1])
    _log(f"   {name}: mean normalized row-sum residual stale/matched: before the cast {pre:.1f}x "
         f"(matched {np.mean(res['matched'][0]):.2e}), after the cast {post:.2f}x "
         f"(stale {np.mean(res['stale'][1]):.3e}, matched {np.mean(res['matched'][1]):.3e})")
    assert post > 1.0


@pytest.mark.parametrize("name", ["gqa_8k", "gqa_64k"])
def test_saved_output_deltas_every_row(name):
    """The stale and dO-matched corrections at full size, every row, as properties of the kernel's
    inputs: delta_i = sum_k dO_ik O_ik (bf16 dO) and sum_k dO^_ik O_ik (dO^ decoded from its E5M2 codes
    and block scales, codes the quantize tests check bit for bit), evaluated in float64 from the same O
    the kernel is given.  Bound: FP32 accumulation, 2^-20 of sum_k |dO_ik O_ik| (d = 128 terms)."""
    from fp8_attention_amd import api
    w = W.WORKLOADS[name]
    inputs = W.generate(w)
    do = inputs["do"].cuda()
    B, Hq, L, D = w.batch, w.heads_q, w.seqlen, w.d_v
    shape = api.AttnShape(B, Hq, w.heads_kv, L, w.d_qk, D, w.causal)
    # any FP32 O of the right shape exercises the pass; a seeded one keeps the forward out of it
    o = torch.randn((B, Hq, L, D), generator=torch.Generator().manual_seed(7), dtype=torch.float32).cuda()
    do_c = api.quantize(do, "cols", "e5m2", api.padded_len(L))
    for mode in ("stale", "do_matched"):
        if mode == "stale":
            got = api.attn_delta(shape, mode, o=o, do=do)
            x = do.double()
        else:
            got = api.attn_delta(shape, mode, o=o, do_c=do_c)
            codes = do_c.codes[..., :L, :].view(torch.float8_e5m2).double()
            x = codes * do_c.scales[..., :L, :].double().repeat_interleave(32, dim=-1)
        torch.cuda.synchronize()
        prod = x * o.double()
        ref, mag = prod.sum(-1), prod.abs().sum(-1)
        err = (got.double() - ref).abs()
        worst = float((err / mag.clamp_min(1e-300)).max())
        _log(f"   {name} {mode}: max |err| / sum|dO O| = {worst:.2e} over {ref.numel()} rows")
        assert bool((err <= 2.0 ** -20 * mag + 1e-30).all()), worst
        del prod, ref, mag, err, x
