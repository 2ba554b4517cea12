"""CPU checks of the Python binding's argument validation: nothing reaches a kernel
with host memory or an operand whose layout differs from what the kernels read."""
import pytest
import torch

from fp8_attention_amd import api


def test_operand_layouts():
    s = api.AttnShape(2, 4, 2, 200, 192, 128, True)      # Lp = 256
    assert api._op_shapes(s, "q_c") == ((2, 4, 256, 192), (2, 4, 256, 6))
    assert api._op_shapes(s, "q_s") == ((2, 4, 192, 256), (2, 4, 192, 8))
    assert api._op_shapes(s, "k_c") == ((2, 2, 256, 192), (2, 2, 256, 6))
    assert api._op_shapes(s, "k_s") == ((2, 2, 192, 256), (2, 2, 192, 8))
    assert api._op_shapes(s, "v_c") == ((2, 2, 256, 128), (2, 2, 256, 4))
    assert api._op_shapes(s, "v_s") == ((2, 2, 128, 256), (2, 2, 128, 8))
    assert api._op_shapes(s, "do_c") == ((2, 4, 256, 128), (2, 4, 256, 4))
    assert api._op_shapes(s, "do_s") == ((2, 4, 128, 256), (2, 4, 128, 8))


def _cpu_ops(s):
    ops = {}
    for n in ("q_c", "q_s", "k_c", "k_s", "v_c", "v_s", "do_c", "do_s"):
        cs, ss = api._op_shapes(s, n)
        ops[n] = api.Fp8Operand(torch.zeros(cs, dtype=torch.uint8), torch.ones(ss, dtype=torch.float32))
    return ops


@pytest.mark.parametrize("call", ["fwd", "delta_stale", "delta_matched", "bwd", "bwd_dkdv", "bwd_dq", "quantize"])
def test_host_tensors_are_rejected(call):
    s = api.AttnShape(1, 2, 1, 64, 64, 64, True)
    ops = _cpu_ops(s)
    lse = torch.zeros(1, 2, 64)
    o = torch.zeros(1, 2, 64, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        if call == "fwd":
            api.attn_fwd(s, ops["q_c"], ops["k_c"], ops["v_s"])
        elif call == "delta_stale":
            api.attn_delta(s, "stale", o=o, do=o.bfloat16())
        elif call == "delta_matched":
            api.attn_delta(s, "matched", do_c=ops["do_c"], q_c=ops["q_c"], k_c=ops["k_c"], v_c=ops["v_c"], lse=lse)
        elif call == "bwd":
            api.attn_bwd(s, ops, lse, lse)
        elif call == "bwd_dkdv":
            api.attn_bwd_dkdv(s, ops, lse, lse)
        elif call == "bwd_dq":
            api.attn_bwd_dq(s, ops, lse, lse)
        else:
            api.quantize(o)


def test_unknown_delta_mode():
    s = api.AttnShape(1, 1, 1, 64, 64, 64, False)
    with pytest.raises(ValueError, match="unknown delta mode"):
        api.attn_delta(s, "centered", o=torch.zeros(1, 1, 64, 64))
