"""The Python binding refuses caller-supplied outputs of the wrong type, shape or device
before it calls the library: the C ABI receives only pointers, so a wrong tensor would be
written past its end.  CPU only: the library entry point is replaced by a sentinel that
fails the test if it is ever reached."""
import pytest
import torch

import exact_attention_82_amd as ea
from exact_attention_82_amd import _lib


@pytest.fixture
def no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the library was called although the arguments are invalid")
    monkeypatch.setattr(_lib, "load", forbidden)


B, H, S, D = 1, 2, 16, 64


def qkv(dtype=torch.bfloat16):
    return tuple(torch.zeros(B, H, S, D, dtype=dtype) for _ in range(3))


@pytest.mark.parametrize("out,lse", [
    (torch.zeros(B, H, S, D, dtype=torch.bfloat16), None),     # fp32 O expected
    (torch.zeros(B, H, S, D - 1), None),                         # too small
    (torch.zeros(B, H, S + 1, D), None),                         # wrong shape
    (None, torch.zeros(B, H, S, dtype=torch.float64)),           # lse must be fp32
    (None, torch.zeros(B, H, S - 1)),                            # lse too small
])
def test_attn_fwd_refuses_bad_outputs(no_library, out, lse):
    q, k, v = qkv()
    with pytest.raises(ValueError):
        ea.attn_fwd(q, k, v, out=out, lse=lse)


def test_attn_fwd_ex_output_type_must_match(no_library):
    q, k, v = qkv()
    with pytest.raises(ValueError):   # bf16 requested, fp32 tensor given
        ea.attn_fwd_ex(q, k, v, out_dtype=torch.bfloat16, out=torch.zeros(B, H, S, D))
    with pytest.raises(ValueError):   # fp32 requested, bf16 tensor given
        ea.attn_fwd_ex(q, k, v, out_dtype=torch.float32,
                       out=torch.zeros(B, H, S, D, dtype=torch.bfloat16))


def test_varlen_merge_noalloc_and_backward_outputs(no_library):
    q = torch.zeros(H, 40, D, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10, 40], dtype=torch.int32)
    with pytest.raises(ValueError):
        ea.attn_fwd_varlen(q, q, q, cu, cu, 30, 30, out=torch.zeros(H, 39, D))
    with pytest.raises(ValueError):
        ea.attn_fwd_varlen(q, q, q, cu, cu, 30, 30, lse=torch.zeros(H, 40, 1))
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        ea.attn_merge(ws, 2, B, H, S, D, out=torch.zeros(B, H, S, D // 2))
    qq, kk, vv = qkv()
    with pytest.raises(ValueError):
        ea.attn_fwd_splitkv_noalloc(qq, kk, vv, 2, lse=torch.zeros(B, H, 2 * S))
    o, dout, lse = torch.zeros(B, H, S, D), torch.zeros(B, H, S, D), torch.zeros(B, H, S)
    with pytest.raises(ValueError):
        ea.attn_bwd(qq, kk, vv, o, lse, dout, dk=torch.zeros(B, H, S, D, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        ea.attn_bwd(qq, kk, vv, o, lse, dout, dq=torch.zeros(B, H, S - 1, D))


def test_inputs_on_different_devices_are_refused(no_library):
    q, k, v = qkv()
    k = torch.zeros(B, H, S, D, dtype=torch.bfloat16, device="meta")
    with pytest.raises(ValueError):
        ea.attn_fwd(q, k, v)
