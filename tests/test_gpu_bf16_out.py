"""GPU checks of attn_fwd_ex with bf16 output, through the C ABI.

The bf16 O must be exactly the fp32 O of attn_fwd rounded to the nearest bf16 (ties to
even, torch's rounding) -- the same kernel and arithmetic up to the store -- and lse must
be identical; against the fp64 oracle the bf16 O stays within the bf16 bar.  Covers every
kernel mode that writes O: the plain kernel (large grids), the two-group kernel (small
grids), the causal tile-pair kernel, tails in both sequence dimensions, and all input
types and head dims.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_helpers import check, scale_for, upload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import exact_attention_82_amd as ea

CASES = [
    # dtype, B, H, Sq, Sk, d, causal
    ("bf16", 2, 3, 300, 333, 64, False),     # small grid: two-group kernel, tails
    ("bf16", 2, 3, 300, 300, 128, True),
    ("bf16", 1, 4, 257, 513, 256, True),
    ("bf16", 4, 16, 640, 640, 128, False),   # 320 workgroups: plain kernel
    ("bf16", 1, 40, 1024, 1024, 128, True),  # causal tile pairs (320 tiles, 160 pairs)
    ("fp8", 1, 4, 200, 1000, 128, False),
    ("f32", 1, 2, 130, 97, 64, True),
]


@pytest.mark.parametrize("dtype,B,H,Sq,Sk,d,causal", CASES)
def test_bf16_output_is_the_rounded_fp32_output(dtype, B, H, Sq, Sk, d, causal):
    inp = si.make_attention_inputs(B, H, Sq, Sk, d, seed=21, dtype=dtype)
    q, k, v = upload(inp)
    sq, sk, sv = inp.scales
    sc = scale_for(d)
    eff = float(np.float32(sc * sq * sk)) if dtype == "fp8" else sc
    print(f"bf16 out {dtype} B={B} H={H} Sq={Sq} Sk={Sk} d={d} causal={causal} "
          f"kernel={ea.attn_kernel_name(B, H, Sq, Sk, d, int(causal), ea.dtype_code(q))}", flush=True)
    o32, l32 = ea.attn_fwd(q, k, v, scale=eff, causal=causal)
    o16, l16 = ea.attn_fwd_ex(q, k, v, scale=eff, causal=causal, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(l16, l32)
    if dtype == "fp8":
        return  # the fp8 output is in code units (times the v descale); covered by the equality
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, causal)
    check(f"bf16 out {dtype} d={d}", o16.float().cpu().numpy(), l16.cpu().numpy(), ro, rl, "bf16")
