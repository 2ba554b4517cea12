"""Pins of the oracle's FP8 codec and block quantizer (CPU only).

Pinned against: torch's float8_e4m3fn / float8_e5m2 casts (a library routine,
round-to-nearest-even), the formats' closed-form constants, brute force over
scale exponents, and invariants (power-of-two equivariance, half-ulp error).
"""
import numpy as np
import pytest
import torch

from oracle import fp8

TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_decode_table_matches_torch(name):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TORCH[name]).to(torch.float64).numpy()
    got = fp8.decode_table(name)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_closed_form_constants():
    d4, d5 = fp8.decode_table("e4m3"), fp8.decode_table("e5m2")
    assert d4[0x7E] == 448.0 and np.isnan(d4[0x7F]) and d4[0x01] == 2.0 ** -9
    assert d4[0x08] == 2.0 ** -6 and d4[0x38] == 1.0 and d4[0xB8] == -1.0
    assert d5[0x7B] == 57344.0 and d5[0x7C] == np.inf and np.isnan(d5[0x7D])
    assert d5[0x01] == 2.0 ** -16 and d5[0x3C] == 1.0
    assert np.nanmax(np.abs(d4[np.isfinite(d4)])) == fp8.E4M3.fmax
    assert np.nanmax(np.abs(d5[np.isfinite(d5)])) == fp8.E5M2.fmax


def _all_bf16_as_f32():
    bits = (np.arange(65536, dtype=np.uint32) << 16)
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_encode_exhaustive_bf16_times_scales(name):
    """Every finite bf16 value times 2**k (k in [-24, 24]) that lies in range encodes like torch."""
    fmt = fp8.FORMATS[name]
    base = _all_bf16_as_f32()
    for k in range(-24, 25, 3):
        x = base.astype(np.float64) * 2.0 ** k       # exact: a power-of-two multiple of a bf16
        x = x[np.abs(x) <= fmt.fmax].astype(np.float32)
        ref = torch.from_numpy(x).to(TORCH[name]).view(torch.uint8).numpy()
        got = fp8.encode(x.astype(np.float64), fmt)
        bad = np.nonzero(ref != got)[0]
        assert bad.size == 0, (k, x[bad[:5]], ref[bad[:5]], got[bad[:5]])


def test_round_half_even_and_sign():
    e4 = fp8.E4M3
    # midpoint between 1.0 (m=0) and 1.125 (m=1) goes to the even mantissa 1.0
    assert fp8.encode(np.array([1.0 + 1 / 16]), e4)[0] == 0x38
    # midpoint between 1.125 (m=1) and 1.25 (m=2) goes to 1.25
    assert fp8.encode(np.array([1.0 + 3 / 16]), e4)[0] == 0x3A
    # half the smallest subnormal rounds to zero (even), 3/2 of it to 2 * 2**-9
    assert fp8.encode(np.array([2.0 ** -10]), e4)[0] == 0x00
    assert fp8.encode(np.array([1.5 * 2.0 ** -9]), e4)[0] == 0x02
    # sign is kept for values that round to zero
    assert fp8.encode(np.array([-1e-9]), e4)[0] == 0x80
    assert fp8.encode(np.array([-0.0]), e4)[0] == 0x80
    with pytest.raises(ValueError):
        fp8.encode(np.array([449.0]), e4)


def _k_brute(amax, fmax):
    if amax == 0:
        return -126
    for k in range(-126, 128):
        if amax <= fmax * 2.0 ** k:
            return k
    raise AssertionError


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_scale_exponent_brute_force(name):
    fmt = fp8.FORMATS[name]
    rng = np.random.default_rng(3)
    vals = list(np.exp(rng.uniform(-90, 90, 1500)))
    for k in range(-140, 120, 7):        # boundaries: Fmax * 2**k, its neighbours, powers of two
        b = fmt.fmax * 2.0 ** k
        vals += [b, np.nextafter(b, 0), np.nextafter(b, np.inf), 2.0 ** k]
    vals += [0.0, 2.0 ** -149, 1e-45, 3.0e38]
    vals = np.array(vals)
    got = fp8.scale_exponent(vals, fmt)
    ref = np.array([_k_brute(v, fmt.fmax) for v in vals])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_block_quantizer_invariants(name):
    fmt = fp8.FORMATS[name]
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    x = x.astype(np.float64)
    codes, s, dec = fp8.quantize_lastaxis(x, fmt)
    xb = x.reshape(64, 8, 32)
    # the scale is minimal and keeps every element in range
    am = np.abs(xb).max(-1)
    assert np.all(am <= fmt.fmax * s) and np.all(am > fmt.fmax * s / 2)
    # decode(encode) equals the decoded values, and the error is at most half a grid step
    assert np.array_equal(fp8.dequantize_lastaxis(codes, s, fmt), dec)
    v = np.abs(xb / s[..., None])
    step = np.ldexp(1.0, np.maximum(np.frexp(v)[1] - 1, fmt.emin) - fmt.mbits)
    assert np.all(np.abs(dec.reshape(64, 8, 32) - xb) <= 0.5 * step * s[..., None])
    # power-of-two equivariance: same codes, scales times 2**m
    for m in (-5, 3, 11):
        c2, s2, _ = fp8.quantize_lastaxis(x * 2.0 ** m, fmt)
        assert np.array_equal(c2, codes) and np.array_equal(s2, s * 2.0 ** m)
    # an all-zero block takes the clamped scale 2**-126 and zero codes
    c0, s0, _ = fp8.quantize_lastaxis(np.zeros((1, 32)), fmt)
    assert s0[0, 0] == 2.0 ** -126 and not c0.any()


def test_cast_ambiguity_bound_covers_perturbed_casts():
    """Any value within the error bound casts to a value within ``delta`` of the exact cast."""
    rng = np.random.default_rng(11)
    for fmt in (fp8.E4M3, fp8.E5M2):
        x = rng.standard_normal((200, 128)) * np.exp(rng.uniform(-3, 3, (200, 1)))
        err = np.abs(x) * 10.0 ** rng.uniform(-6, -2, x.shape)
        dec, delta, nflag, nblock = fp8.cast_lastaxis(x, fmt, err)
        assert nflag > 0
        for _ in range(20):
            xp = x + err * rng.uniform(-1, 1, x.shape)
            decp, _, _, _ = fp8.cast_lastaxis(xp, fmt)
            assert np.all(np.abs(decp - dec) <= delta + 1e-300)
    # a block whose amax sits on a scale boundary is flagged
    xb = np.zeros((1, 32))
    xb[0, 0] = 448.0 * 2.0 ** -8
    xb[0, 1] = 1.3 * 2.0 ** -17      # subnormal at scale 2**-8: its cast depends on the scale
    _, delta, _, nblock = fp8.cast_lastaxis(xb, fp8.E4M3, np.full_like(xb, 1e-9))
    assert nblock == 1 and delta[0, 1] > 0
