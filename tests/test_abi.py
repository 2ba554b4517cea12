"""CPU checks of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments with the documented status before touching the GPU.

Every call here carries at least one invalid argument, so none of them can
reach a kernel launch even on a machine with a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

from fp8_attention_amd import _lib
from fp8_attention_amd.api import AttnShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dm_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libdm.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(dm_\w+)\s*\(", text, flags=re.M)))


def test_header_declarations_are_exported():
    names = _declared()
    assert set(names) == set(_lib.EXPORTS), names
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= syms


def test_padded_len_and_strings():
    lib = _lib.load()
    assert [lib.dm_padded_len(x) for x in (0, 1, 128, 129, 65536)] == [0, 128, 128, 256, 65536]
    assert lib.dm_padded_len(-1) == -1
    for s in range(7):
        assert _lib.status_string(s).startswith("DM_")
    assert "unknown" in _lib.status_string(99)


FAKE = 0x1000          # aligned, never dereferenced: every call below fails validation first
MIS = 0x1004


def _op(p=FAKE, q=FAKE):
    return _lib.Operand(p, q)


def _fwd(shape, q=None, o=FAKE, lse=FAKE):
    lib = _lib.load()
    s = shape.c() if isinstance(shape, AttnShape) else shape
    return lib.dm_attn_fwd(ctypes.byref(s) if s is not None else None, q or _op(), _op(), _op(), o, lse, None)


BAD_SHAPES = [
    AttnShape(1, 3, 2, 128, 128, 128, True),       # Hq % Hkv != 0
    AttnShape(1, 2, 2, 128, 96, 128, True),        # unsupported d_qk
    AttnShape(1, 2, 2, 128, 128, 192, True),       # unsupported d_v
    AttnShape(1, 2, 2, 128, 256, 128, True),       # d_qk = 256 only with d_v = 256
    AttnShape(1, 2, 2, 128, 128, 256, True),       # d_v = 256 only with d_qk = 256
    AttnShape(0, 2, 2, 128, 128, 128, True),       # empty batch
    AttnShape(1, 2, 2, -5, 128, 128, True),        # negative length
    AttnShape(1, 2, 2, 128, 128, 128, True, -1.0),  # non-positive scale
    AttnShape(1, 2, 2, 128, 128, 128, True, float("nan")),
    AttnShape(1, 2, 2, (1 << 26) + 1, 128, 128, True),
    AttnShape(1, 2, 2, _lib.DM_MAX_SEQLEN + 1, 128, 128, True),   # beyond the 32-bit load offsets
]


@pytest.mark.parametrize("shape", BAD_SHAPES)
def test_bad_shapes(shape):
    assert _fwd(shape) == _lib.DM_ERR_SHAPE


def test_longest_sequence_passes_the_shape_check():
    """L = DM_MAX_SEQLEN is accepted by the shape check (the call then fails on its NULL output,
    which is checked after the shape), one more is not; the header states the same limit."""
    longest = AttnShape(1, 2, 2, _lib.DM_MAX_SEQLEN, 128, 128, True)
    assert _fwd(longest, o=None) == _lib.DM_ERR_NULL
    assert _fwd(AttnShape(1, 2, 2, _lib.DM_MAX_SEQLEN + 1, 128, 128, True), o=None) == _lib.DM_ERR_SHAPE
    m = re.search(r"#define DM_MAX_SEQLEN \(1 << (\d+)\)", open(HEADER).read())
    assert m and (1 << int(m.group(1))) == _lib.DM_MAX_SEQLEN
    # the d = 128 dK/dV kernel addresses up to 127 channel rows of Lp bytes with 32-bit offsets
    assert 127 * _lib.DM_MAX_SEQLEN + 128 * 16 < 2 ** 31


def test_bad_causal_flag_and_null_shape():
    s = AttnShape(1, 2, 2, 128, 128, 128, True).c()
    s.causal = 2
    assert _fwd(s) == _lib.DM_ERR_SHAPE
    assert _fwd(None) == _lib.DM_ERR_NULL


def test_null_and_misaligned_pointers():
    # a NULL output with an otherwise valid call is caught; so is a misaligned one
    good = AttnShape(1, 2, 2, 128, 128, 128, True)
    assert _fwd(good, o=None) == _lib.DM_ERR_NULL
    assert _fwd(good, q=_op(FAKE, None)) == _lib.DM_ERR_NULL
    assert _fwd(good, lse=MIS) == _lib.DM_ERR_ALIGN
    assert _fwd(good, q=_op(MIS, FAKE)) == _lib.DM_ERR_ALIGN


def test_delta_mode_and_required_pointers():
    lib = _lib.load()
    s = AttnShape(1, 2, 2, 128, 128, 128, True).c()
    n = _lib.Operand(None, None)
    assert lib.dm_attn_delta(ctypes.byref(s), 7, FAKE, FAKE, n, n, n, n, FAKE, FAKE, None) == _lib.DM_ERR_ENUM
    # stale needs o and dO; matched needs the four operands and lse
    assert lib.dm_attn_delta(ctypes.byref(s), 0, None, FAKE, n, n, n, n, None, FAKE, None) == _lib.DM_ERR_NULL
    assert lib.dm_attn_delta(ctypes.byref(s), 1, FAKE, None, n, n, n, n, None, FAKE, None) == _lib.DM_ERR_NULL
    assert lib.dm_attn_delta(ctypes.byref(s), 2, None, None, _op(), _op(), _op(), n, FAKE, FAKE,
                             None) == _lib.DM_ERR_NULL
    assert lib.dm_attn_delta(ctypes.byref(s), 2, None, None, _op(), _op(), _op(), _op(), None, FAKE,
                             None) == _lib.DM_ERR_NULL


def test_bwd_probe_pointers_come_in_pairs():
    lib = _lib.load()
    s = AttnShape(1, 2, 2, 128, 128, 128, True).c()
    ops = [_op()] * 7
    assert lib.dm_attn_bwd(ctypes.byref(s), *ops, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.DM_ERR_NULL
    assert lib.dm_attn_bwd(ctypes.byref(s), *ops, FAKE, FAKE, FAKE, FAKE, FAKE, MIS, MIS, None) == _lib.DM_ERR_ALIGN
    s.d_v = 32
    assert lib.dm_attn_bwd(ctypes.byref(s), *ops, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == _lib.DM_ERR_SHAPE


def test_split_backward_validation():
    lib = _lib.load()
    s = AttnShape(1, 2, 2, 128, 128, 128, True).c()
    op = _op()
    assert lib.dm_attn_bwd_dkdv(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, None, None) == _lib.DM_ERR_NULL
    assert lib.dm_attn_bwd_dkdv(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, MIS, None) == _lib.DM_ERR_ALIGN
    assert lib.dm_attn_bwd_dq(ctypes.byref(s), *[op] * 5, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.DM_ERR_NULL
    assert lib.dm_attn_bwd_dq(ctypes.byref(s), *[op] * 5, FAKE, FAKE, MIS, None, None, None) == _lib.DM_ERR_ALIGN
    # the three-probe dQ call requires every probe buffer
    pr = lib.dm_attn_bwd_dq_probes
    assert pr(ctypes.byref(s), *[op] * 5, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.DM_ERR_NULL
    assert pr(ctypes.byref(s), *[op] * 5, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == _lib.DM_ERR_NULL
    assert pr(ctypes.byref(s), *[op] * 5, FAKE, FAKE, FAKE, FAKE, FAKE, MIS, None) == _lib.DM_ERR_ALIGN
    # the dK/dV probe call requires both probe buffers
    kp = lib.dm_attn_bwd_dkdv_probes
    assert kp(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == _lib.DM_ERR_NULL
    assert kp(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.DM_ERR_NULL
    assert kp(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, FAKE, MIS, None) == _lib.DM_ERR_ALIGN
    s.d_qk = 96
    assert pr(ctypes.byref(s), *[op] * 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE
    assert kp(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE
    assert lib.dm_attn_bwd_dkdv(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE
    assert lib.dm_attn_bwd_dq(ctypes.byref(s), *[op] * 5, FAKE, FAKE, FAKE, None, None, None) == _lib.DM_ERR_SHAPE


def _expected_split_bytes(B, Hq, Hkv, L, d_qk, d_v):
    """The head-split policy as documented: d_qk = d_v = 128 only; the query heads of a KV group
    are dealt to 2, 4, ... workgroups per 128-key tile while the grid has fewer than 1024
    workgroups and the split divides the group; partial dK and dV sums of 4 bytes per channel."""
    if (d_qk, d_v) != (128, 128) or L == 0:
        return 0
    G, nwg, hs = Hq // Hkv, -(-L // 128) * Hkv * B, 1
    while G % (2 * hs) == 0 and nwg * hs < 1024:
        hs *= 2
    return 0 if hs == 1 else hs * B * Hkv * L * (d_qk + d_v) * 4


@pytest.mark.parametrize("dims", [(2, 16, 4, 4096, 128, 128), (4, 32, 8, 8192, 128, 128), (1, 16, 4, 65536, 128, 128),
                                  (1, 8, 1, 192, 128, 128), (1, 4, 2, 320, 128, 128), (1, 6, 2, 1000, 128, 128),
                                  (1, 1, 1, 1, 128, 128), (3, 64, 1, 128, 128, 128), (1, 8, 8, 100, 128, 128),
                                  (2, 16, 4, 4096, 256, 256), (2, 16, 16, 4096, 192, 128), (1, 4, 1, 0, 128, 128)])
def test_head_split_workspace_size(dims):
    lib = _lib.load()
    s = AttnShape(*dims, True).c()
    n = ctypes.c_int64(-1)
    assert lib.dm_attn_bwd_dkdv_workspace_size(ctypes.byref(s), ctypes.byref(n)) == _lib.DM_OK
    assert n.value == _expected_split_bytes(*dims), (dims, n.value)
    assert n.value < 256 << 20
    assert lib.dm_attn_bwd_dkdv_workspace_size(ctypes.byref(s), None) == _lib.DM_ERR_NULL
    assert lib.dm_attn_bwd_dkdv_workspace_size(None, ctypes.byref(n)) == _lib.DM_ERR_NULL
    s.d_v = 96
    assert lib.dm_attn_bwd_dkdv_workspace_size(ctypes.byref(s), ctypes.byref(n)) == _lib.DM_ERR_SHAPE


def test_head_split_entry_validation():
    lib = _lib.load()
    s = AttnShape(2, 16, 4, 4096, 128, 128, True).c()
    n = ctypes.c_int64(0)
    lib.dm_attn_bwd_dkdv_workspace_size(ctypes.byref(s), ctypes.byref(n))
    need = n.value
    assert need == 4 * 2 * 4 * 4096 * 256 * 4
    op = _op()
    ws = lib.dm_attn_bwd_dkdv_ws
    assert ws(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, None, need, None) == _lib.DM_ERR_NULL
    assert ws(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, MIS, need, None) == _lib.DM_ERR_ALIGN
    assert ws(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == _lib.DM_ERR_WORKSPACE
    assert ws(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, None, FAKE, need, None) == _lib.DM_ERR_NULL
    s.d_qk = 96
    assert ws(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == _lib.DM_ERR_SHAPE


def test_noalloc_entry_validation():
    """The allocation-free dK/dV call: argument errors, and a shape whose head split needs more
    than the fixed scratch is refused before any GPU call."""
    lib = _lib.load()
    na = lib.dm_attn_bwd_dkdv_noalloc
    op = _op()
    s = AttnShape(1, 16, 8, 12288, 128, 128, True).c()      # 768 key tiles x heads: split 2, 192 MiB
    n = ctypes.c_int64(0)
    assert lib.dm_attn_bwd_dkdv_workspace_size(ctypes.byref(s), ctypes.byref(n)) == _lib.DM_OK
    assert n.value == 192 << 20 > _lib.DM_NOALLOC_SCRATCH_BYTES
    assert na(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, None) == _lib.DM_ERR_WORKSPACE
    assert na(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, None, None) == _lib.DM_ERR_NULL
    assert na(ctypes.byref(s), *[op] * 6, FAKE, FAKE, MIS, FAKE, None) == _lib.DM_ERR_ALIGN
    assert na(None, *[op] * 6, FAKE, FAKE, FAKE, FAKE, None) == _lib.DM_ERR_NULL
    s.d_qk = 96
    assert na(ctypes.byref(s), *[op] * 6, FAKE, FAKE, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE
    # the 4K GQA workload's split fits exactly
    s = AttnShape(2, 16, 4, 4096, 128, 128, True).c()
    assert lib.dm_attn_bwd_dkdv_workspace_size(ctypes.byref(s), ctypes.byref(n)) == _lib.DM_OK
    assert n.value == _lib.DM_NOALLOC_SCRATCH_BYTES


def test_quantize_validation():
    lib = _lib.load()
    q = lib.dm_quantize_blockfp8
    assert q(FAKE, 2, 1, 64, 64, 64, 0, 0, FAKE, FAKE, None) == _lib.DM_ERR_ENUM      # dtype
    assert q(FAKE, 0, 1, 64, 64, 64, 5, 0, FAKE, FAKE, None) == _lib.DM_ERR_ENUM      # axis
    assert q(FAKE, 0, 1, 64, 64, 64, 0, 3, FAKE, FAKE, None) == _lib.DM_ERR_ENUM      # format
    assert q(FAKE, 0, 1, 64, 48, 64, 0, 0, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE     # cols % 32
    assert q(FAKE, 0, 1, 64, 48, 64, 1, 0, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE     # cols % 32 (rows axis)
    assert q(FAKE, 0, 1, 64, 64, 32, 0, 0, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE     # rows_out < rows
    assert q(FAKE, 0, 1, 64, 64, 80, 1, 0, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE     # rows_out % 32 (rows axis)
    assert q(FAKE, 0, 0, 64, 64, 64, 0, 0, FAKE, FAKE, None) == _lib.DM_ERR_SHAPE     # batch
    assert q(None, 0, 1, 64, 64, 64, 0, 0, FAKE, FAKE, None) == _lib.DM_ERR_NULL
    assert q(FAKE, 0, 1, 64, 64, 64, 0, 0, FAKE, MIS, None) == _lib.DM_ERR_ALIGN
