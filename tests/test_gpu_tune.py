"""Shape-keyed tuning on the GPU: every legal launch plan of a shape meets the parity bar
against the oracle; attn_tune picks one of them, stores it for the shape, and later
attn_fwd calls of that shape are bit-identical to a call with that plan set explicitly
(attn_plan_set), which is also how a choice is carried to another run.  Split-count
tuning likewise: attn_splitkv_num_splits then returns the tuned count and the split path
with that count reproduces the tuned result bit for bit."""
import numpy as np
import pytest
import torch

import exact_attention_82_amd as ea
import synthetic_inputs as si
from tests.gpu_helpers import check, oracle_rows, scale_for, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def clean_plan_table():
    ea.attn_plan_clear()
    yield
    ea.attn_plan_clear()


def _np(t):
    return t.detach().float().cpu().numpy()


def test_every_plan_is_correct_and_the_tuned_call_reproduces_its_plan():
    B, H, S, d = 1, 4, 1000, 128   # causal bf16: plain (head groups 1/2/4), complementary,
    inp = si.make_attention_inputs(B, H, S, S, d, seed=71, dtype="bf16", hot_row_frac=0.01)
    q, k, v = upload(inp)           # tile pairs and two-group plans are all legal here
    sc = scale_for(d)
    ro, rl = oracle_rows(inp, sc, True)
    rule = ea.attn_plan_get(B, H, S, S, d, 1, ea.ATTN_BF16)
    results = {}
    for plan in range(28):
        try:
            ea.attn_plan_set(B, H, S, S, d, 1, ea.ATTN_BF16, plan)
        except ea.AttnError:
            continue
        o, lse = ea.attn_fwd(q, k, v, scale=sc, causal=True)
        torch.cuda.synchronize()
        s, g = ea.plan_parts(plan)
        print(f"plan {plan} (schedule {s}, head group {g}) kernel "
              f"{ea.attn_kernel_name(B, H, S, S, d, 1, ea.ATTN_BF16)}", flush=True)
        check(f"plan {plan}", _np(o).reshape(B * H, S, d), _np(lse).reshape(B * H, S), ro, rl, "bf16")
        results[plan] = (o.clone(), lse.clone())
    assert len(results) == 8 and rule in results
    ea.attn_plan_clear()
    o_t = torch.empty(B, H, S, d, device=q.device)
    l_t = torch.empty(B, H, S, device=q.device)
    best = ea.attn_tune(q, k, v, scale=sc, causal=True, reps=5, out=o_t, lse=l_t)
    assert best in results
    assert ea.attn_plan_get(B, H, S, S, d, 1, ea.ATTN_BF16) == best
    # the outputs attn_tune leaves, a later call, and the explicitly set plan agree bit for bit
    o2, l2 = ea.attn_fwd(q, k, v, scale=sc, causal=True)
    torch.cuda.synchronize()
    for a, b in ((o_t, o2), (l_t, l2), (o2, results[best][0]), (l2, results[best][1])):
        assert torch.equal(a, b)
    # another shape is untouched by the stored plan
    assert ea.attn_plan_get(B, H, S, S + 1, d, 1, ea.ATTN_BF16) == ea.attn_plan_get(B, H, S, S + 1, d, 1, ea.ATTN_BF16)


def test_split_count_tuning():
    B, H, Sq, Sk, d = 1, 8, 128, 8192, 128
    inp = si.make_attention_inputs(B, H, Sq, Sk, d, seed=72, dtype="fp8")
    q, k, v = upload(inp)
    sc = scale_for(d)
    desc = tuple(float(x) for x in inp.scales)
    rule = ea.attn_splitkv_num_splits(B, H, Sq, Sk, d, ea.ATTN_FP8_E4M3)
    o_t = torch.empty(B, H, Sq, d, device=q.device)
    l_t = torch.empty(B, H, Sq, device=q.device)
    n = ea.attn_tune_splitkv(q, k, v, scale=sc, descales=desc, reps=5, out=o_t, lse=l_t)
    print(f"split count: rule {rule}, tuned {n}", flush=True)
    assert n >= 1 and (n & (n - 1) == 0 or n == rule)
    assert ea.attn_splitkv_num_splits(B, H, Sq, Sk, d, ea.ATTN_FP8_E4M3) == n
    ws = ea.attn_fwd_splitkv(q, k, v, n, scale=sc, descales=desc)
    o, lse = ea.attn_merge(ws, n, B, H, Sq, d)
    torch.cuda.synchronize()
    assert torch.equal(o, o_t) and torch.equal(lse, l_t)
    ro, rl = oracle_rows(inp, sc, False)
    check(f"tuned split n={n}", _np(o).reshape(B * H, Sq, d), _np(lse).reshape(B * H, Sq), ro, rl, "fp8")
    ea.attn_plan_clear()
    assert ea.attn_splitkv_num_splits(B, H, Sq, Sk, d, ea.ATTN_FP8_E4M3) == rule
