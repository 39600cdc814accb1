"""attn_fwd_splitkv_noalloc (the split-KV call whose chunk states live in the library's
static device array) against the same split through attn_fwd_splitkv + attn_merge with a
caller workspace: identical results, on two calls in a row, the second with a smaller
input (a different workspace layout inside the same array, over the first call's
leftover contents).  Both also meet the parity bar against the oracle."""
import numpy as np
import pytest
import torch

import exact_attention_82_amd as ea
import synthetic_inputs as si
from tests.gpu_helpers import check, oracle_rows, scale_for, upload

pytestmark = pytest.mark.gpu

CALLS = [
    # (dtype, B, H, Sq, Sk, d, num_splits, causal, seed): the fp8 split workload's heads and
    # query rows with a quarter of its keys, then a smaller bf16 call with a causal mask
    ("fp8", 1, 8, 128, 8192, 128, 16, 0, 61),
    ("bf16", 1, 2, 100, 1000, 64, 3, 1, 62),
]


def _run(case):
    dt, B, H, Sq, Sk, d, n, causal, seed = case
    inp = si.make_attention_inputs(B, H, Sq, Sk, d, seed=seed, dtype=dt)
    q, k, v = upload(inp)
    scale = scale_for(d)
    desc = tuple(float(x) for x in inp.scales)
    print(f"noalloc case dtype={dt} B={B} H={H} Sq={Sq} Sk={Sk} d={d} n={n} causal={causal}", flush=True)
    o1, l1 = ea.attn_fwd_splitkv_noalloc(q, k, v, n, scale=scale, causal=bool(causal), descales=desc)
    ws = ea.attn_fwd_splitkv(q, k, v, n, scale=scale, causal=bool(causal), descales=desc)
    o2, l2 = ea.attn_merge(ws, n, B, H, Sq, d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), float((o1 - o2).abs().max())
    assert torch.equal(l1, l2)
    rows = np.arange(Sq) if Sq <= 128 else None
    ro, rl = oracle_rows(inp, scale, bool(causal), rows=rows)
    got_o = o1.cpu().numpy().reshape(B * H, Sq, d)
    got_l = l1.cpu().numpy().reshape(B * H, Sq)
    check(f"noalloc {dt} n={n}", got_o, got_l, ro, rl, dt)


def test_noalloc_matches_the_workspace_split_on_two_calls_in_a_row():
    for case in CALLS:
        _run(case)
