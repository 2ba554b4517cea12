"""How the scaled FP8 matrix instructions accumulate, measured on the GPU.

The Delta-Matching project page (section 01, "What changes in FP8?") takes the
FP8 products to accumulate in FP32.  The oracle's parity allowance assumes more:
one FP8 instruction's result may sit up to GAMMA * sum_k |a_k b_k| from the exact
dot product (oracle/attention.py).  This file measures that, on the exact forms
the kernels issue, through a test-only probe library (tests/hip/mfma_acc.hip)
that reaches the instruction through the kernels' own wrappers and lane layouts:

* v_mfma_scale_f32_32x32x64_f8f6f4 and v_mfma_scale_f32_16x16x128_f8f6f4;
* the format pairs the kernels use (E4M3 x E4M3 for S and P V, E4M3 x E5M2 and
  E5M2 x E4M3 for dP, dV, dQ, dK);
* contraction lengths 64 .. 256 (chained instructions, as over d = 128 or a
  128-key step);
* a zero accumulator input, and a nonzero one (the dP products that start from
  -delta);
* operands drawn like the attention workloads (RMSNorm'd Q and K with the
  long-context channel gains, V, dO, softmax-shaped P and dS) and operands that
  span the full finite code range with spread block scales.

Expected values are FP64 dot products of the decoded codes (the oracle's codec).
Asserted, per output element:
  * zero accumulator input: |result - exact| <= GAMMA * sum|ab|, over chains of 1 to
    32 instructions (the error does not grow with the chain);
  * accumulator input C: |result - (C + exact)| <= GAMMA * sum|ab| + 2^-20 |result|,
    i.e. C is carried at FP32 precision and does not pass through the products'
    narrow adder (a C comparable to the products, like -delta, adds nothing beyond
    the result's own rounding, which the oracle's TAU covers);
  * the largest error is far above what an exactly rounded FP32 dot product could
    produce, so the allowance is needed at all.
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "hip", "libmfma_acc.so")
FMT = {"e4m3": 0, "e5m2": 1}


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


_lib = None


def _probe_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run `python fp8_attention_amd/build.py`")
        _lib = ctypes.CDLL(LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        _lib.mfma_acc_probe.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, i32, vp]
        _lib.mfma_acc_probe.restype = i32
    return _lib


def run_probe(form, fa, fb, a_codes, a_exp, b_codes, b_exp, c_in):
    """GPU result of the chained instruction over [T, rows, K] operands (rows = form)."""
    T, rows, K = a_codes.shape
    assert rows == form and b_codes.shape == (T, rows, K)
    assert a_exp.shape == b_exp.shape == (T, rows, K // 32) and c_in.shape == (T, rows, rows)
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()   # noqa: E731
    ta, tea = dev(a_codes, torch.uint8), dev(a_exp, torch.uint8)
    tb, teb = dev(b_codes, torch.uint8), dev(b_exp, torch.uint8)
    tc = dev(c_in.astype(np.float32), torch.float32)
    out = torch.empty_like(tc)
    st = _probe_lib().mfma_acc_probe(form, FMT[fa], FMT[fb], ta.data_ptr(), tea.data_ptr(), tb.data_ptr(),
                                     teb.data_ptr(), tc.data_ptr(), out.data_ptr(), T, K,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def decode(codes, exps, fmt):
    """FP64 values of codes [T, rows, K] with exponent bytes [T, rows, K/32]."""
    vals = fp8.decode_table(fmt)[codes]
    sc = np.exp2(np.repeat(exps.astype(np.float64) - 127.0, 32, axis=-1))
    return vals * sc


def quantized(x, fmt):
    """Block-quantize x [T, rows, K] along K with the oracle: codes and exponent bytes."""
    codes, scales, _ = fp8.quantize_lastaxis(x, fmt)
    exps = (np.log2(scales) + 127).astype(np.uint8)
    return codes.astype(np.uint8), exps


def tiles(x, rows):
    """[N, K] -> [N // rows, rows, K] (N a multiple of rows)."""
    return x.reshape(-1, rows, x.shape[-1])


# ---------------------------------------------------------------------------
# operand sets
# ---------------------------------------------------------------------------

def _attention_rows(n, d, seed):
    """RMSNorm'd rows with channel 7 scaled (the long-context Q/K gains), V ~ N(0,1), dO ~ N(0, 0.01)."""
    g = np.random.default_rng(seed)
    def rms(x, gain):
        y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6)
        y[..., 7] *= gain
        return y
    q = rms(g.standard_normal((n, d)), 2.0)
    k = rms(g.standard_normal((n, d)), 5.4)
    v = g.standard_normal((n, d))
    do = 0.1 * g.standard_normal((n, d))
    return q, k, v, do


def _softmax_rows(n, m, seed, temp=3.0):
    """Softmax-shaped rows [n, m] (P) and a dS-shaped companion P * (x - mean)."""
    g = np.random.default_rng(seed)
    s = temp * g.standard_normal((n, m))
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    x = g.standard_normal((n, m))
    ds = p * (x - (p * x).sum(axis=1, keepdims=True))
    return p, ds


def _full_range(T, rows, K, fmt, seed):
    """Every finite code with equal probability, exponent bytes 127 +- 20 per block."""
    g = np.random.default_rng(seed)
    table = fp8.decode_table(fmt)
    finite = np.flatnonzero(np.isfinite(table)).astype(np.uint8)
    codes = g.choice(finite, size=(T, rows, K))
    exps = (127 + g.integers(-20, 21, size=(T, rows, K // 32))).astype(np.uint8)
    return codes, exps


def operand_cases():
    """(name, form, fa, fb, a_codes, a_exp, b_codes, b_exp) for every product shape the kernels form."""
    cases = []
    n, d = 512, 128
    q, k, v, do = _attention_rows(n, d, 5)
    p, ds = _softmax_rows(n, 256, 6)
    pt, dst = _softmax_rows(256, n, 7)
    for form in (32, 16):
        # products over channels: S = Q K^T, dP = dO V^T (d = 128; 64 with one 32x32x64 instruction)
        qc, qe = quantized(tiles(q, form), "e4m3")
        kc, ke = quantized(tiles(k, form), "e4m3")
        vc, ve = quantized(tiles(v, form), "e4m3")
        dc, de = quantized(tiles(do, form), "e5m2")
        cases.append((f"S{form}", form, "e4m3", "e4m3", qc, qe, kc, ke))
        if form == 32:
            cases.append((f"dP{form}", form, "e4m3", "e5m2", vc, ve, dc, de))      # A = V, B = dO
            cases.append((f"S{form}_k64", form, "e4m3", "e4m3", qc[..., :64], qe[..., :2], kc[..., :64], ke[..., :2]))
        else:
            cases.append((f"dP{form}", form, "e5m2", "e4m3", dc, de, vc, ve))      # A = dO, B = V
        # products over the sequence: P V (A = V^<s> rows, B = P rows), dV (A = dO^<s>, B = P),
        # dQ (A = K^<s>, B = dS), dK (A = Q^<s>, B = dS), 256-long
        vs, vse = quantized(tiles(np.ascontiguousarray(v[:256].T), form), "e4m3")
        dos, dose = quantized(tiles(np.ascontiguousarray(do[:256].T), form), "e5m2")
        ks, kse = quantized(tiles(np.ascontiguousarray(k[:256].T), form), "e4m3")
        qs, qse = quantized(tiles(np.ascontiguousarray(q[:256].T), form), "e4m3")
        T = vs.shape[0]
        pc, pe = quantized(tiles(p[:T * form], form), "e4m3")
        dsc_, dse = quantized(tiles(ds[:T * form], form), "e5m2")
        pqc, pqe = quantized(tiles(pt[:T * form, :256], form), "e4m3")
        dqc, dqe = quantized(tiles(dst[:T * form, :256], form), "e5m2")
        cases.append((f"PV{form}", form, "e4m3", "e4m3", vs, vse, pc, pe))
        cases.append((f"dV{form}", form, "e5m2", "e4m3", dos, dose, pqc, pqe))
        cases.append((f"dQ{form}", form, "e4m3", "e5m2", ks, kse, dsc_, dse))
        cases.append((f"dK{form}", form, "e4m3", "e5m2", qs, qse, dqc, dqe))
        # full range of finite codes, both format pairs
        for fa, fb in (("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")):
            K = 128 if form == 32 else 256
            ac, ae = _full_range(64, form, K, fa, 11 + form)
            bc, be = _full_range(64, form, K, fb, 12 + form)
            cases.append((f"full{form}_{fa}x{fb}", form, fa, fb, ac, ae, bc, be))
    return cases


def _exact(case):
    name, form, fa, fb, ac, ae, bc, be = case
    a, b = decode(ac, ae, fa), decode(bc, be, fb)
    return np.einsum("tik,tjk->tij", a, b), np.einsum("tik,tjk->tij", np.abs(a), np.abs(b))


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------

def _chain_cases():
    """P V-shaped (softmax-shaped P) and same-sign full-range products over 512 and 2048 (8 to 32
    chained instructions)."""
    out = []
    for K in (512, 2048):
        p, _ = _softmax_rows(128, K, 60 + K)
        v = np.random.default_rng(61 + K).standard_normal((K, 128))
        for form in (32, 16):
            vs, vse = quantized(tiles(np.ascontiguousarray(v.T), form), "e4m3")
            pc, pe = quantized(tiles(p[:vs.shape[0] * form], form), "e4m3")
            out.append((f"PV{form}_k{K}", form, "e4m3", "e4m3", vs, vse, pc, pe))
            ac, ae = _full_range(16, form, K, "e4m3", 62 + K)
            bc, be = _full_range(16, form, K, "e4m3", 63 + K)
            out.append((f"fullpos{form}_k{K}", form, "e4m3", "e4m3", ac & 0x7F, ae, bc & 0x7F, be))
    return out


def test_zero_accumulator_within_gamma_and_beyond_fp32():
    worst_all, rows = 0.0, []
    for case in operand_cases() + _chain_cases():
        name, form, fa, fb, ac, ae, bc, be = case
        exact, sabs = _exact(case)
        got = run_probe(form, fa, fb, ac, ae, bc, be, np.zeros_like(exact))
        err = np.abs(got - exact)
        ok = sabs > 0
        ratio = np.where(ok, err / np.where(ok, sabs, 1.0), 0.0)
        worst = float(ratio.max())
        med = float(np.median(ratio[ok & (err > 0)])) if np.any(ok & (err > 0)) else 0.0
        # an exactly rounded FP32 result of each chained instruction would be within
        # 2^-24 of |partial| per instruction, summed: (K / instruction K) * 2^-24 * sum|ab|
        nk = ac.shape[-1] // (64 if form == 32 else 128)
        fp32_bound = nk * 2.0 ** -24
        frac_beyond = float(np.mean(ratio > fp32_bound))
        rows.append((name, worst, med, frac_beyond))
        _log(f"   {name:22s} max|err|/sum|ab| = 2^{np.log2(max(worst, 1e-300)):6.2f}  median(nonzero) "
             f"2^{np.log2(max(med, 1e-300)):6.2f}  beyond exact-FP32 rounding: {100 * frac_beyond:5.1f}%")
        assert np.all(err <= A.GAMMA * sabs), (name, worst)
        worst_all = max(worst_all, worst)
    # the allowance is needed: errors reach far beyond FP32 rounding (2^-24 per instruction)
    assert worst_all > 2.0 ** -18, worst_all


def test_nonzero_accumulator_input():
    """The dP products that start from -delta: C enters the instruction as its accumulator input.
    The error stays within GAMMA * sum|ab| plus a few FP32 ulps of the result for C from 1e-3 to
    1e6 times sum|ab|, a delta-like C (minus the row mean) and a cancelling C (minus the product):
    C does not pass through the narrow adder of the products."""
    g = np.random.default_rng(31)
    summary = {}
    for case in operand_cases():
        name, form, fa, fb, ac, ae, bc, be = case
        if not (name.startswith("dP") or name.startswith("full") or name.startswith("S")):
            continue
        exact, sabs = _exact(case)
        for cname, c in (
                # like -delta: minus a weighted mean of the row's products (comparable to the entries)
                ("mean", -np.mean(exact, axis=2, keepdims=True) * (1 + 0.1 * g.standard_normal(exact.shape))),
                # cancelling the product: the result is a small difference
                ("cancel", -exact * (1 + 2.0 ** -10 * g.standard_normal(exact.shape))),
                ("x1e3", 1e3 * sabs * g.standard_normal(exact.shape)),
                ("x1e6", 1e6 * sabs * g.standard_normal(exact.shape)),
                ("x1e-3", 1e-3 * sabs * g.standard_normal(exact.shape))):
            c = c.astype(np.float32).astype(np.float64)
            got = run_probe(form, fa, fb, ac, ae, bc, be, c)
            want = c + exact
            err = np.abs(got - want)
            bound = A.GAMMA * sabs + 2.0 ** -20 * np.abs(got)
            ok2 = sabs > 0
            r_prod = float(np.max(np.where(ok2, err / np.where(ok2, sabs, 1.0), 0.0)))
            r_bound = float(np.max(err / np.maximum(bound, 1e-300)))
            summary[(name, cname)] = r_bound
            _log(f"   {name:22s} C={cname:6s} max|err|/sum|ab| = 2^{np.log2(max(r_prod, 1e-300)):7.2f}  "
                 f"max|err| / (GAMMA sum|ab| + 2^-20 |result|) = {r_bound:.3f}")
            assert np.all(err <= bound), (name, cname, r_bound)
    _log(f"   worst fraction of the bound over {len(summary)} cases: {max(summary.values()):.3f}")


def test_long_chains():
    """2048 chained instructions, as many as accumulate one dK or dV element of a key tile at the
    64K context shape (4 query heads x 65536 queries / 128 per instruction): softmax-shaped P
    times V-shaped rows, and same-sign full-range codes; the error stays within GAMMA sum|ab|."""
    for form in (16, 32):
        K = 2048 * (128 if form == 16 else 64)
        g = np.random.default_rng(70 + form)
        p, _ = _softmax_rows(form, K, 71 + form, temp=2.0)
        v = g.standard_normal((form, K))
        pc, pe = quantized(p[None], "e4m3")
        vc, ve = quantized(v[None], "e4m3")
        ac, ae = _full_range(1, form, K, "e4m3", 72 + form)
        bc, be = _full_range(1, form, K, "e4m3", 73 + form)
        for name, case in (("PV", (vc, ve, pc, pe)), ("fullpos", (ac & 0x7F, ae, bc & 0x7F, be))):
            a_c, a_e, b_c, b_e = case
            a, b = decode(a_c, a_e, "e4m3"), decode(b_c, b_e, "e4m3")
            exact = np.einsum("tik,tjk->tij", a, b)
            sabs = np.einsum("tik,tjk->tij", np.abs(a), np.abs(b))
            got = run_probe(form, "e4m3", "e4m3", a_c, a_e, b_c, b_e, np.zeros_like(exact))
            r = float(np.max(np.abs(got - exact) / sabs))
            _log(f"   {name}{form} over 2048 chained instructions: max|err|/sum|ab| = 2^{np.log2(r):.2f}")
            assert np.all(np.abs(got - exact) <= A.GAMMA * sabs), (name, form, r)


def test_instruction_shapes_agree_only_within_gamma():
    """The same contraction through 2 x 32x32x64 and 1 x 16x16x128 (over 128 channels) gives
    results within GAMMA of each other; the fraction that is bit-identical is reported
    (the backward kernels use both shapes for S and dP)."""
    q, k, v, do = _attention_rows(512, 128, 41)
    same = tot = 0
    for x, y, fx, fy in ((q, k, "e4m3", "e4m3"), (do, v, "e5m2", "e4m3")):
        # 16x16 tiles of [32-row block] products: build both shapes over the same row pairs
        xc, xe = quantized(tiles(x, 32), fx)
        yc, ye = quantized(tiles(y, 32), fy)
        r32 = run_probe(32, fx, fy, xc, xe, yc, ye, np.zeros((xc.shape[0], 32, 32)))
        # the 16-row sub-tiles (rows 0-15 and 16-31 of each side) through the 16x16x128 form
        sub = lambda c, i: c[:, 16 * i:16 * i + 16]     # noqa: E731
        for i in range(2):
            for j in range(2):
                r16 = run_probe(16, fx, fy, sub(xc, i), sub(xe, i), sub(yc, j), sub(ye, j),
                                np.zeros((xc.shape[0], 16, 16)))
                ref = r32[:, 16 * i:16 * i + 16, 16 * j:16 * j + 16]
                same += int(np.sum(r16 == ref))
                tot += r16.size
                a = decode(sub(xc, i), sub(xe, i), fx)
                b = decode(sub(yc, j), sub(ye, j), fy)
                sabs = np.einsum("tik,tjk->tij", np.abs(a), np.abs(b))
                assert np.all(np.abs(r16 - ref) <= 2 * A.GAMMA * sabs)
    _log(f"   bit-identical between the two shapes: {same} of {tot} ({100.0 * same / tot:.1f}%)")
