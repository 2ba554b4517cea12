"""FP8 codec and power-of-two block quantizer of the CPU oracle (FP64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module.

What it follows
---------------
* "Delta-Matching for reliable FP8 attention training", section 01, sub-heading
  "What changes in FP8?": the hatted operands are decoded FP8 values *including
  their block scales*.  The page names no block size and no scale rule; the
  readings used here are

  - one scale per 32 consecutive elements along the contraction axis of the
    matmul the operand feeds (1x32 blocks);
  - the scale is the power of two 2**k with the smallest integer k such that
    amax <= Fmax * 2**k (amax = largest magnitude in the block), k clamped to
    [-126, 127] so the scale is a normal float32; an all-zero block takes
    k = -126.  With this rule x / 2**k never exceeds Fmax, so no saturation
    rule is ever needed;
  - elements are rounded to the nearest FP8 value, ties to even, subnormals
    kept, sign kept (a negative value that rounds to zero encodes as 0x80).

* The formats are the OCP 8-bit floating-point formats (the news article on the
  project names E4M3 for the forward operands and E5M2 for the gradients):
  E4M3FN -- 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities,
  S.1111.111 is NaN, largest finite 448, smallest subnormal 2**-9;
  E5M2 -- 1 sign, 5 exponent (bias 15), 2 mantissa bits, IEEE-style inf/NaN,
  largest finite 57344, smallest subnormal 2**-16.

Everything is exact in FP64: scaling by a power of two and rounding onto a
power-of-two-spaced grid introduce no error of their own.
"""
from __future__ import annotations

import dataclasses

import numpy as np

BLOCK = 32
K_MIN, K_MAX = -126, 127


@dataclasses.dataclass(frozen=True)
class Format:
    name: str
    ebits: int
    mbits: int
    bias: int
    fmax: float
    ieee_specials: bool  # True: all-ones exponent encodes inf/NaN (E5M2)

    @property
    def emin(self) -> int:          # unbiased exponent of the smallest normal
        return 1 - self.bias

    @property
    def sub_step(self) -> float:    # spacing of the subnormal grid
        return 2.0 ** (self.emin - self.mbits)


E4M3 = Format("e4m3", 4, 3, 7, 448.0, False)
E5M2 = Format("e5m2", 5, 2, 15, 57344.0, True)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2}


def fmt_of(f) -> Format:
    return f if isinstance(f, Format) else FORMATS[f]


def decode_table(fmt) -> np.ndarray:
    """Value (FP64) of each of the 256 codes, NaN/inf where the format says so."""
    fmt = fmt_of(fmt)
    out = np.empty(256, dtype=np.float64)
    emask = (1 << fmt.ebits) - 1
    mmask = (1 << fmt.mbits) - 1
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> fmt.mbits) & emask
        m = c & mmask
        if e == emask and fmt.ieee_specials:
            out[c] = sign * np.inf if m == 0 else np.nan
        elif e == emask and m == mmask and not fmt.ieee_specials:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * m * fmt.sub_step
        else:
            out[c] = sign * (1.0 + m / (1 << fmt.mbits)) * 2.0 ** (e - fmt.bias)
    return out


def _grid_exponent(a: np.ndarray, fmt: Format) -> np.ndarray:
    """Unbiased exponent of the binade that holds |a| (subnormals share emin)."""
    _, e = np.frexp(a)               # a = f * 2**e, f in [0.5, 1)
    return np.maximum(e - 1, fmt.emin)


def _pow2(k: np.ndarray) -> np.ndarray:
    """2.0**k for integer k in the FP64 normal range, built from the exponent field."""
    return ((np.asarray(k, dtype=np.int64) + 1023) << 52).view(np.float64)


def round_to_grid(v: np.ndarray, fmt) -> np.ndarray:
    """Nearest FP8 value of v (ties to even), as FP64.  Requires |v| <= Fmax.

    The grid step at |v| is 2^(u - mbits), u the binade exponent of |v| (never below
    the format's emin, where the subnormals share one step); |v| / step is scaled by
    an exact power of two and rounded half-to-even."""
    fmt = fmt_of(fmt)
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > fmt.fmax):
        raise ValueError("value outside the format's finite range")
    # unbiased FP64 exponent field of a (FP64 zeros and subnormals give -1023 and so emin)
    u = np.maximum((a.view(np.int64) >> 52) - 1023, fmt.emin)
    q = np.rint(a * _pow2(fmt.mbits - u))         # exact scaling; np.rint rounds half to even
    return np.copysign(q * _pow2(u - fmt.mbits), v)


def encode(v: np.ndarray, fmt) -> np.ndarray:
    """FP8 codes (uint8) of v, round-to-nearest-even.  Requires |v| <= Fmax."""
    fmt = fmt_of(fmt)
    v = np.asarray(v, dtype=np.float64)
    r = np.abs(round_to_grid(v, fmt))
    u = _grid_exponent(r, fmt)
    frac = np.ldexp(r, -u)                        # in [0, 2)
    normal = frac >= 1.0
    mant_scale = 1 << fmt.mbits
    m = np.where(normal, (frac - 1.0) * mant_scale, frac * mant_scale)
    e_field = np.where(normal, u + fmt.bias, 0)
    code = (e_field.astype(np.int64) << fmt.mbits) | m.astype(np.int64)
    code |= np.signbit(v).astype(np.int64) << 7
    return code.astype(np.uint8)


def decode(codes: np.ndarray, fmt) -> np.ndarray:
    return decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def scale_exponent(amax: np.ndarray, fmt) -> np.ndarray:
    """Smallest integer k with amax <= Fmax * 2**k, clamped to [-126, 127].

    With amax = f * 2**E and Fmax = g * 2**G (f, g in [0.5, 1)), the answer is
    E - G when f <= g and E - G + 1 otherwise.
    """
    fmt = fmt_of(fmt)
    amax = np.asarray(amax, dtype=np.float64)
    f, e = np.frexp(amax)
    g, ge = np.frexp(fmt.fmax)
    k = e - ge + (f > g).astype(np.int64)
    k = np.where(amax == 0, K_MIN, k)
    return np.clip(k, K_MIN, K_MAX).astype(np.int64)


def quantize_lastaxis(x: np.ndarray, fmt):
    """Block-quantize along the last axis (length a multiple of 32).

    Returns (codes uint8 like x, scales float64 [..., n/32], decoded FP64 like x).
    """
    fmt = fmt_of(fmt)
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (n // BLOCK, BLOCK))
    k = scale_exponent(np.abs(xb).max(axis=-1), fmt)
    s = np.ldexp(1.0, k)
    v = xb / s[..., None]
    codes = encode(v, fmt).reshape(x.shape)
    dec = (round_to_grid(v, fmt) * s[..., None]).reshape(x.shape)
    return codes, s, dec


def dequantize_lastaxis(codes: np.ndarray, scales: np.ndarray, fmt) -> np.ndarray:
    codes = np.asarray(codes)
    n = codes.shape[-1]
    d = decode(codes, fmt).reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    return (d * np.asarray(scales, dtype=np.float64)[..., None]).reshape(codes.shape)


# ---------------------------------------------------------------------------
# In-kernel casts and their ambiguity.
#
# Casts of FP32 values that the kernel itself computed (probabilities, score
# gradients) cannot be reproduced bit for bit: the kernel's FP32 value differs
# from the exact FP64 value by rounding.  When the exact value lies within that
# rounding error of an FP8 rounding midpoint, or its block amax lies within it
# of a scale boundary, two different casts are both correct.  ``cast_lastaxis``
# returns the cast of the exact value plus, per element, the largest change of
# the decoded value that any cast of a value inside [x - err, x + err] can give.
# ---------------------------------------------------------------------------

def _cast_with_scale(xb, s, fmt):
    v = np.clip(xb / s, -fmt.fmax, fmt.fmax)
    return round_to_grid(v, fmt) * s


def cast_lastaxis(x: np.ndarray, fmt, err: np.ndarray | None = None):
    """Block cast along the last axis.

    Returns (decoded, delta, n_elem_flag, n_block_flag); ``delta`` is None when
    ``err`` is None.  ``err`` is an elementwise non-negative absolute bound of
    how far the kernel's value may be from ``x``.
    """
    fmt = fmt_of(fmt)
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    shp = x.shape[:-1] + (n // BLOCK, BLOCK)
    xb = x.reshape(shp)
    a = np.abs(xb)
    k = scale_exponent(a.max(axis=-1), fmt)
    s = np.ldexp(1.0, k)[..., None]
    dec = _cast_with_scale(xb, s, fmt)
    if err is None:
        return dec.reshape(x.shape), None, 0, 0
    eb = np.asarray(err, dtype=np.float64).reshape(shp)
    lo = _cast_with_scale(xb - eb, s, fmt)
    hi = _cast_with_scale(xb + eb, s, fmt)
    delta = np.maximum(np.abs(hi - dec), np.abs(dec - lo))
    n_elem = int(np.count_nonzero(delta))
    # Scale ambiguity: the kernel's block amax lies in [amax_lo, amax_hi].
    k_lo = scale_exponent(np.maximum(a - eb, 0.0).max(axis=-1), fmt)
    k_hi = scale_exponent((a + eb).max(axis=-1), fmt)
    flag = k_lo != k_hi
    n_block = int(np.count_nonzero(flag))
    if n_block:
        # every scale 2^kk with k_lo <= kk <= k_hi of a flagged block is a possible kernel
        # scale: take the largest change any of them gives (block by block, kk = k_lo + o)
        idx = np.nonzero(flag)
        xf, ef, df = xb[idx], eb[idx], dec[idx]
        klo, khi = k_lo[idx], k_hi[idx]
        worst = np.zeros_like(xf)
        for o in range(int((khi - klo).max()) + 1):
            use = np.nonzero(klo + o <= khi)[0]             # blocks with a candidate at this offset
            sa = np.ldexp(1.0, klo[use] + o)[:, None]
            xu, eu, du = xf[use], ef[use], df[use]
            w = worst[use]
            for cand in (_cast_with_scale(xu - eu, sa, fmt), _cast_with_scale(xu, sa, fmt),
                         _cast_with_scale(xu + eu, sa, fmt)):
                w = np.maximum(w, np.abs(cand - du))
            worst[use] = w
        dd = delta[idx]
        delta[idx] = np.maximum(dd, worst)
    return dec.reshape(x.shape), delta.reshape(x.shape), n_elem, n_block


def cast_axis(x: np.ndarray, fmt, axis: int, err: np.ndarray | None = None):
    """``cast_lastaxis`` along an arbitrary axis of a 2-D array."""
    if axis in (-1, x.ndim - 1):
        return cast_lastaxis(x, fmt, err)
    xt = np.swapaxes(x, axis, -1)
    et = None if err is None else np.swapaxes(err, axis, -1)
    dec, delta, ne, nb = cast_lastaxis(np.ascontiguousarray(xt), fmt,
                                       None if et is None else np.ascontiguousarray(et))
    dec = np.swapaxes(dec, axis, -1)
    delta = None if delta is None else np.swapaxes(delta, axis, -1)
    return dec, delta, ne, nb
