"""GPU parity: the HIP library, called through its C ABI, against the fp64 oracle on
the same seeded, rounded inputs.

Covers the worked example of the pages (full softmax and the split-KV workspace
states), the five workload configurations (full comparison where the oracle is quick,
sampled rows at full size otherwise), ragged shapes that span several tiles with tails
in both sequence dimensions, causal alignment for Sq != Sk, fully masked rows, split
counts with empty chunks, and the degenerate cases.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_helpers import check, oracle_rows, sample_rows, scale_for, to_device, upload, TOL

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import exact_attention_82_amd as ea

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DT_CODE = {"f32": 0, "bf16": 1, "fp8": 2}
# Largest lag (log2 units) of a stored chunk reference behind the chunk maximum: the bf16
# main loop moves its reference only when a lane's probability sum would pass 2^33, the
# guarded loop (and fp32) when a score passes the reference by 8; fp8 keeps every
# 2^4-scaled probability at or below E4M3's largest value 448.
LAG_LOG2 = {"bf16": 33.0, "f32": 8.0, "fp8": math.log2(448.0) - 4.0}


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def _run_fwd(inp, scale, causal):
    """attn_fwd on the stored inputs; for fp8 the q/k descales are folded into the
    scale and O is multiplied by the v descale, as the entry point documents."""
    q, k, v = upload(inp)
    sq, sk, sv = inp.scales
    eff = float(np.float32(scale * sq * sk)) if inp.dtype == "fp8" else scale
    o, lse = ea.attn_fwd(q, k, v, scale=eff, causal=causal)
    o = _np(o)
    return (o * np.float32(sv) if inp.dtype == "fp8" else o), _np(lse)


def _run_split(inp, scale, causal, n, descales=(1.0, 1.0, 1.0)):
    q, k, v = upload(inp)
    ws = ea.attn_fwd_splitkv(q, k, v, n, scale=scale, causal=causal, descales=descales)
    o, lse = ea.attn_merge(ws, n, inp.B, inp.H, inp.Sq, inp.d)
    return ws, _np(o), _np(lse)


# ------------------------------------------------------------------ worked example
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_worked_example_full_softmax(dtype, d):
    g = _golden("worked_example.json")
    inp = si.worked_example_inputs(d, dtype)
    o, lse = _run_fwd(inp, 1.0, False)
    tol = TOL[dtype]["max_o"]
    print(f"worked example {dtype} d={d}: O={o[0, 0, 0, 0]:.6f} lse={lse[0, 0, 0]:.6f}", flush=True)
    assert abs(o[0, 0, 0, 0] - g["merged_output"]) <= max(tol, 5e-7)
    assert np.all(o[0, 0, 0, 1:] == 0.0)
    ref_o, ref_l = oracle.attention(inp.q64[0, 0], inp.k64[0, 0], inp.v64[0, 0], 1.0)
    assert abs(lse[0, 0, 0] - ref_l[0]) <= (1e-5 if dtype == "f32" else TOL[dtype]["lse"])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_worked_example_split_states_and_merge(dtype):
    g = _golden("worked_example.json")
    inp = si.worked_example_inputs(64, dtype)
    tol = max(TOL[dtype]["max_o"], 5e-7)
    for n in (1, 2, 3, 4):
        ws, o, lse = _run_split(inp, 1.0, False, n)
        assert abs(o[0, 0, 0, 0] - g["merged_output"]) <= tol, (n, o[0, 0, 0, 0])
        assert np.all(o[0, 0, 0, 1:] == 0.0)
        m, l, u = (_np(t) for t in ea.workspace_views(ws, n, 1, 1, 1, 64))
        bounds = oracle.split_bounds(4, n)
        for s, (a, b) in enumerate(bounds):
            if a == b:  # empty chunk: neutral state
                assert np.isneginf(m[s, 0, 0, 0]) and l[s, 0, 0, 0] == 0.0
                assert np.all(u[s, 0, 0, 0] == 0.0)
        if n == 2:
            for s, want in enumerate(g["two_block_split"]):
                print(f"{dtype} block {s}: m={m[s,0,0,0]:.6f} l={l[s,0,0,0]:.6f} "
                      f"u={u[s,0,0,0,0]:.6f}", flush=True)
                assert abs(m[s, 0, 0, 0] - want["m"]) <= 1e-5
                assert abs(l[s, 0, 0, 0] - want["l"]) <= 1e-5
                assert abs(u[s, 0, 0, 0, 0] - want["u"]) <= max(tol, 1e-5)
            # and the merge is not the naive average the page warns about
            assert abs(o[0, 0, 0, 0] - g["naive_average_of_block_outputs"]) > 0.5


# ------------------------------------------------------------------ config 1: tiny fp32
@pytest.mark.parametrize("causal", [False, True])
def test_config1_tiny_fp32(causal):
    inp = si.make_attention_inputs(1, 2, 128, 128, 64, seed=1, dtype="f32")
    sc = scale_for(64)
    o, lse = _run_fwd(inp, sc, causal)
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, causal)
    check(f"c1 causal={causal}", o, lse, ro, rl, "f32")


# ------------------------------------------------------------------ ragged shapes, all dtypes and head dims
RAGGED = [(2, 3, 300, 457), (1, 2, 457, 300), (1, 1, 1, 1), (1, 2, 1, 190), (2, 1, 190, 1),
          (1, 1, 129, 65), (1, 1, 64, 1000)]


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_shapes(dtype, d, causal):
    for i, (B, H, Sq, Sk) in enumerate(RAGGED):
        inp = si.make_attention_inputs(B, H, Sq, Sk, d, seed=100 + i, dtype=dtype)
        sc = scale_for(d)
        o, lse = _run_fwd(inp, sc, causal)
        ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, causal)
        check(f"ragged {dtype} d={d} causal={causal} {(B, H, Sq, Sk)}", o, lse, ro, rl, dtype)


def test_fully_masked_rows_give_zero_and_neg_inf():
    inp = si.make_attention_inputs(1, 2, 200, 70, 128, seed=7, dtype="bf16")
    o, lse = _run_fwd(inp, scale_for(128), True)
    hidden = 200 - 70  # rows i < Sq - Sk see no key under bottom-right alignment
    assert np.all(o[:, :, :hidden] == 0.0)
    assert np.all(np.isneginf(lse[:, :, :hidden]))
    assert np.all(np.isfinite(lse[:, :, hidden:]))


# ------------------------------------------------------------------ config 2 and 3 at full size
def _full_size_sampled(B, H, S, d, seed, causal, nrows):
    inp = si.make_attention_inputs(B, H, S, S, d, seed=seed, dtype="bf16")
    sc = scale_for(d)
    o, lse = _run_fwd(inp, sc, causal)
    rows = sample_rows(S, nrows, seed)
    rng = np.random.default_rng(seed + 1)
    heads = sorted({0, B * H - 1} | set(rng.choice(B * H, size=min(B * H, 6), replace=False).tolist()))
    ro, rl = oracle_rows(inp, sc, causal, rows=rows, heads=heads)
    og = o.reshape(B * H, S, d)[heads][:, rows]
    lg = lse.reshape(B * H, S)[heads][:, rows]
    check(f"B={B} H={H} S={S} d={d} causal={causal} (sampled)", og, lg, ro, rl, "bf16")
    return o


@pytest.mark.parametrize("causal", [False, True])
def test_config2_full_size_sampled(causal):
    _full_size_sampled(8, 32, 2048, 64, 2, causal, 160)


@pytest.mark.parametrize("causal", [False, True])
def test_config3_full_size_sampled(causal):
    _full_size_sampled(1, 8, 8192, 128, 3, causal, 160)


def test_config3_values_of_ones_give_ones():
    """Property at full size: with V = 1 every output element is 1 (rows sum to 1)."""
    inp = si.make_attention_inputs(1, 8, 8192, 8192, 128, seed=3, dtype="bf16")
    q, k, _ = upload(inp)
    ones = torch.ones_like(k)
    for causal in (False, True):
        o, lse = ea.attn_fwd(q, k, ones, scale=scale_for(128), causal=causal)
        err = float((o - 1.0).abs().max())
        print(f"V=1 causal={causal}: max|O-1|={err:.3e}", flush=True)
        assert err <= 1e-2


# ------------------------------------------------------------------ config 4: head-dim / tail sweep
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("S", [512, 1000, 2048])
@pytest.mark.parametrize("B", [1, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_config4_sweep(d, S, B, causal):
    H = 16
    seed = 400 + (d // 64) * 100 + S // 100 + B
    inp = si.make_attention_inputs(B, H, S, S, d, seed=seed, dtype="bf16", hot_row_frac=0.01)
    sc = scale_for(d)
    o, lse = _run_fwd(inp, sc, causal)
    hot = inp.hot_rows
    heads = sorted(set((hot // S).tolist()[:8]) | {0, B * H - 1})
    hot_rows_in = [int(r % S) for r in hot if (r // S) in heads]
    rows = sample_rows(S, 96, seed, must=hot_rows_in)
    ro, rl = oracle_rows(inp, sc, causal, rows=rows, heads=heads)
    og = o.reshape(B * H, S, d)[heads][:, rows]
    lg = lse.reshape(B * H, S)[heads][:, rows]
    check(f"c4 d={d} S={S} B={B} causal={causal}", og, lg, ro, rl, "bf16")


# ------------------------------------------------------------------ config 5: fp8 split-KV
@pytest.mark.parametrize("n", [1, 4, 16, "auto"])
def test_config5_fp8_splitkv(n):
    if n == "auto":  # the count attn_splitkv_num_splits picks for this shape (32 on 256 CUs)
        n = ea.attn_splitkv_num_splits(1, 8, 128, 32768, 128, ea.ATTN_FP8_E4M3)
        assert n >= 1
    inp = si.make_attention_inputs(1, 8, 128, 32768, 128, seed=5, dtype="fp8")
    sc = scale_for(128)
    ws, o, lse = _run_split(inp, sc, False, n, descales=inp.scales)
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, False)
    check(f"c5 fp8 n={n}", o, lse, ro, rl, "fp8")
    # the chunk states themselves against the oracle's split states (head 0, a few rows).
    # A state (m, l, u) is defined up to its reference: (m + t, l e^-t, u e^-t) merges the
    # same way, and the kernel's reference may lag the chunk maximum; what is fixed is the
    # chunk's log-sum-exp m + ln l and its normalised average u / l.
    m, l, u = (_np(t) for t in ea.workspace_views(ws, n, 1, 8, 128, 128))
    states = oracle.split_states(inp.q64[0, 0, :4], inp.k64[0, 0], inp.v64[0, 0], sc, n)
    for s, (sm, sl, su) in enumerate(states):
        mg, lg, ug = m[s, 0, 0, :4].astype(np.float64), l[s, 0, 0, :4], u[s, 0, 0, :4]
        assert np.all(mg >= sm - LAG_LOG2['fp8'] * math.log(2) - 1e-4) and np.all(mg <= sm + 1e-4)
        np.testing.assert_allclose(mg + np.log(lg), sm + np.log(sl), atol=1e-3)
        np.testing.assert_allclose(ug / lg[:, None], su / sl[:, None], atol=5e-2)


# fp8 with hot query rows (scaled by 4): their scores pass the running reference by more
# than the lag allows on tiles in the middle of a sweep, so the main loop's redo
# (reference moved to the tile's maximum, accumulator and sums rescaled) runs on full
# tiles, in the direct and the split kernels, one and two groups, with a tail tile.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_hot_rows_direct_and_split(d, causal):
    inp = si.make_attention_inputs(1, 4, 300, 2500, d, seed=31 + d, dtype="fp8",
                                   hot_row_frac=0.05, hot_scale=4.0)
    sc = scale_for(d)
    sq, sk, sv = inp.scales
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, causal)
    q, k, v = upload(inp)
    o, lse = ea.attn_fwd(q, k, v, scale=float(np.float32(sc * sq * sk)), causal=causal)
    check(f"fp8 hot rows d={d} causal={causal} attn_fwd", _np(o) * sv, _np(lse), ro, rl, "fp8")
    for n in (1, 3, 8):
        _, o2, l2 = _run_split(inp, sc, causal, n, descales=inp.scales)
        check(f"fp8 hot rows d={d} causal={causal} split n={n}", o2, l2, ro, rl, "fp8")


# Rows scaled by 30 give scores around 100-150: O stays within the fp8 bars, while lse
# carries the score's accumulation error in the 64-deep E4M3 MFMA, measured at about
# 1.5e-5 of |lse| (the fp32 path on the same values: 4.5e-5 absolute), so the absolute
# 1e-3 bar holds only up to |lse| of about 60; this test checks O and that relative bound.
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_large_scores_lse_relative(d):
    inp = si.make_attention_inputs(1, 4, 300, 2500, d, seed=31 + d, dtype="fp8", hot_row_frac=0.05)
    sc = scale_for(d)
    sq, sk, sv = inp.scales
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, False)
    q, k, v = upload(inp)
    o, lse = ea.attn_fwd(q, k, v, scale=float(np.float32(sc * sq * sk)), causal=False)
    loose = dict(TOL["fp8"], lse=float("inf"))
    check(f"fp8 large scores d={d}", _np(o) * sv, _np(lse), ro, rl, "fp8", tol=loose)
    rel = np.abs(_np(lse).astype(np.float64) - rl) / np.maximum(np.abs(rl), 1.0)
    print(f"fp8 large scores d={d}: max |dlse|/|lse| = {rel.max():.3e}", flush=True)
    assert rel.max() <= 3e-5


def test_config5_fp8_direct_forward_with_folded_descales():
    inp = si.make_attention_inputs(1, 8, 128, 32768, 128, seed=5, dtype="fp8")
    sc = scale_for(128)
    sq, sk, sv = inp.scales
    q, k, v = upload(inp)
    o, lse = ea.attn_fwd(q, k, v, scale=float(np.float32(sc * sq * sk)), causal=False)
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, False)
    check("c5 fp8 attn_fwd", _np(o) * sv, _np(lse), ro, rl, "fp8")


# ------------------------------------------------------------------ split-KV on other dtypes and masks


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_counts_with_empty_chunks(dtype, causal):
    inp = si.make_attention_inputs(2, 2, 150, 333, 128, seed=9, dtype=dtype)
    sc = scale_for(128)
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, causal)
    for n in (1, 2, 3, 4, 7, 16, 400):  # 400 > Sk: most chunks are empty
        ws, o, lse = _run_split(inp, sc, causal, n)
        check(f"split {dtype} causal={causal} n={n}", o, lse, ro, rl, dtype)
        # the chunk states of head (0, 0), every row, against the oracle's: empty or fully
        # masked chunks are exactly neutral; otherwise the reference lies within the lag
        # bound below the chunk maximum, and what does not depend on it -- the chunk's
        # log-sum-exp m + ln l and its normalised average u / l -- matches.
        m, l, u = (_np(t).astype(np.float64) for t in ea.workspace_views(ws, n, 2, 2, 150, 128))
        states = oracle.split_states(inp.q64[0, 0], inp.k64[0, 0], inp.v64[0, 0], sc, n, causal)
        tol_u = 1e-2 if dtype == "bf16" else 1e-5
        for s, (sm, sl, su) in enumerate(states):
            mg, lg, ug = m[s, 0, 0], l[s, 0, 0], u[s, 0, 0]
            empty = np.isneginf(sm)
            assert np.array_equal(np.isneginf(mg), empty), (n, s)
            assert np.all(lg[empty] == 0.0) and np.all(ug[empty] == 0.0), (n, s)
            full = ~empty
            if not full.any():
                continue
            lag = LAG_LOG2[dtype] * math.log(2)
            assert np.all(mg[full] <= sm[full] + 1e-4), (n, s)
            assert np.all(mg[full] >= sm[full] - lag - 1e-4), (n, s)
            np.testing.assert_allclose(mg[full] + np.log(lg[full]), sm[full] + np.log(sl[full]),
                                       atol=1e-3)
            np.testing.assert_allclose(ug[full] / lg[full, None], su[full] / sl[full, None],
                                       atol=tol_u)


# ------------------------------------------------------------------ causal schedules
def test_causal_tile_pairs_plan_and_parity():
    """A causal bf16 grid with more tiles than CUs whose tile pairs fit one workgroup per
    CU runs the pair kernel (two groups per workgroup split each pair's keys and merge);
    a grid of at most one tile per CU runs two groups per tile instead.  Parity of the
    pair kernel (set explicitly on the small grid): odd tile count (the middle tile pairs
    with itself), Sq != Sk, ragged last tile."""
    B, H, Sq, Sk, d = 1, 3, 1100, 1500, 128
    nqt = -(-Sq // 128)
    assert ea.attn_kernel_name(1, 40, Sq, Sk, d, 1, ea.ATTN_BF16).startswith("attn_fwd_causal_pairs_bf16_d128")
    assert ea.attn_block_m(1, 40, Sq, Sk, d, 1, ea.ATTN_BF16) == 256
    assert ea.attn_num_workgroups(1, 40, Sq, Sk, d, 1, ea.ATTN_BF16) == 40 * ((nqt + 1) // 2)
    assert ea.attn_kernel_name(B, H, Sq, Sk, d, 1, ea.ATTN_BF16).startswith("attn_fwd_dual_bf16_d128")
    inp = si.make_attention_inputs(B, H, Sq, Sk, d, seed=21, dtype="bf16", hot_row_frac=0.01)
    sc = scale_for(d)
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, True)
    try:
        ea.attn_plan_set(B, H, Sq, Sk, d, 1, ea.ATTN_BF16, 2)
        assert ea.attn_kernel_name(B, H, Sq, Sk, d, 1, ea.ATTN_BF16).startswith("attn_fwd_causal_pairs_bf16_d128")
        assert ea.attn_num_workgroups(B, H, Sq, Sk, d, 1, ea.ATTN_BF16) == B * H * ((nqt + 1) // 2)
        o, lse = _run_fwd(inp, sc, True)
    finally:
        ea.attn_plan_clear()
    check("causal pairs bf16 (1, 3, 1100, 1500)", o, lse, ro, rl, "bf16")
    o, lse = _run_fwd(inp, sc, True)   # the rule's plan: two groups per tile
    check("causal two groups bf16 (1, 3, 1100, 1500)", o, lse, ro, rl, "bf16")


@pytest.mark.parametrize("B,H,Sq,Sk", [(1, 2, 1100, 1500), (2, 1, 900, 700), (1, 3, 1024, 1024)])
def test_causal_tile_pairs_head_dim_64(B, H, Sq, Sk):
    """The d = 64 pair kernel (64-key tiles), set explicitly: odd and even tile counts,
    Sq > Sk (rows with no visible key at the top), Sq < Sk, ragged last tile, and tile
    ranges whose key-tile counts are and are not multiples of the ring's four stages."""
    d = 64
    inp = si.make_attention_inputs(B, H, Sq, Sk, d, seed=40 + Sq % 97, dtype="bf16", hot_row_frac=0.01)
    sc = scale_for(d)
    ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, True)
    nqt = -(-Sq // 128)
    try:
        ea.attn_plan_set(B, H, Sq, Sk, d, 1, ea.ATTN_BF16, 2)
        assert ea.attn_kernel_name(B, H, Sq, Sk, d, 1, ea.ATTN_BF16).startswith("attn_fwd_causal_pairs_bf16_d64")
        assert ea.attn_num_workgroups(B, H, Sq, Sk, d, 1, ea.ATTN_BF16) == B * H * ((nqt + 1) // 2)
        o, lse = _run_fwd(inp, sc, True)
    finally:
        ea.attn_plan_clear()
    check(f"causal pairs bf16 d=64 {(B, H, Sq, Sk)}", o, lse, ro, rl, "bf16")


def test_small_grids_run_two_groups_per_workgroup():
    """Grids of at most one workgroup per CU split each tile's keys between two groups
    (the split-KV chunks too); parity of those kernels is covered by every small-shape
    test above, this pins the choice."""
    assert ea.attn_kernel_name(1, 2, 300, 300, 128, 0, ea.ATTN_BF16).startswith("attn_fwd_dual_bf16_d128")
    assert ea.attn_kernel_name(1, 8, 128, 32768, 128, 0, ea.ATTN_FP8_E4M3, 16).startswith("attn_fwd_splitkv_dual_fp8_d128")
    assert ea.attn_kernel_name(1, 8, 8192, 8192, 128, 0, ea.ATTN_BF16) == "attn_fwd_bf16_d128_bm128_bn32"
    inp = si.make_attention_inputs(1, 2, 300, 333, 128, seed=24, dtype="bf16", hot_row_frac=0.02)
    sc = scale_for(128)
    for causal in (False, True):
        o, lse = _run_fwd(inp, sc, causal)
        ro, rl = oracle.attention(inp.q64, inp.k64, inp.v64, sc, causal)
        check(f"two groups bf16 causal={causal}", o, lse, ro, rl, "bf16")


def test_causal_schedules_without_pairs():
    """fp8 (no pair kernel): complementary tiles per CU when the grid is resident at
    once; bf16 with a grid larger than one workgroup per CU: longest sweeps first."""
    for (B, H, S, d, dtype, seed) in ((1, 2, 700, 64, "fp8", 22), (4, 40, 700, 64, "bf16", 23)):
        adt = ea.ATTN_FP8_E4M3 if dtype == "fp8" else ea.ATTN_BF16
        assert not ea.attn_kernel_name(B, H, S, S, d, 1, adt).startswith("attn_fwd_causal_pairs")
        assert ea.attn_num_workgroups(B, H, S, S, d, 1, adt) == B * H * -(-S // 128)
        inp = si.make_attention_inputs(B, H, S, S, d, seed=seed, dtype=dtype)
        sc = scale_for(d)
        o, lse = _run_fwd(inp, sc, True)
        rows = sample_rows(S, 64, seed)
        heads = [0, B * H // 2, B * H - 1]
        ro, rl = oracle_rows(inp, sc, True, rows=rows, heads=heads)
        og = o.reshape(B * H, S, d)[heads][:, rows]
        lg = lse.reshape(B * H, S)[heads][:, rows]
        check(f"causal {dtype} {(B, H, S, d)}", og, lg, ro, rl, dtype)


# ------------------------------------------------------------------ hygiene
def test_repeat_runs_are_bitwise_identical():
    inp = si.make_attention_inputs(2, 4, 700, 700, 128, seed=11, dtype="bf16")
    q, k, v = upload(inp)
    for causal in (False, True):
        a = ea.attn_fwd(q, k, v, causal=causal)
        b = ea.attn_fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_outputs_do_not_write_past_their_end():
    inp = si.make_attention_inputs(1, 3, 257, 300, 64, seed=12, dtype="bf16")
    q, k, v = upload(inp)
    n_o, n_l, pad = 3 * 257 * 64, 3 * 257, 4096
    o_buf = torch.full((n_o + pad,), float("nan"), device="cuda")
    l_buf = torch.full((n_l + pad,), float("nan"), device="cuda")
    o = o_buf[:n_o].view(1, 3, 257, 64)
    lse = l_buf[:n_l].view(1, 3, 257)
    ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(o_buf[n_o:]).all() and torch.isnan(l_buf[n_l:]).all()
    assert not torch.isnan(o).any()


def test_refused_calls_leave_outputs_untouched():
    inp = si.make_attention_inputs(1, 1, 64, 64, 64, seed=13, dtype="bf16")
    q, k, v = upload(inp)
    o = torch.full((1, 1, 64, 64), 7.0, device="cuda")
    lse = torch.full((1, 1, 64), 7.0, device="cuda")
    lib = ea._lib.load()
    s = torch.cuda.current_stream().cuda_stream
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr()]
    assert lib.attn_fwd(*args, 1, 1, 64, 64, 96, 0.125, 0, 1, s) == 4      # head dim 96
    assert lib.attn_fwd(*args, 1, 1, 64, 64, 64, -1.0, 0, 1, s) == 7      # scale < 0
    assert lib.attn_fwd(*args, 1, 1, 64, 64, 64, 0.125, 2, 1, s) == 7     # causal = 2
    assert lib.attn_fwd(*args, 1, 1, 0, 64, 64, 0.125, 0, 1, s) == 2      # Sq = 0
    assert lib.attn_fwd(*args, 1, 1, 64, 64, 64, 0.125, 0, 9, s) == 4     # dtype 9
    torch.cuda.synchronize()
    assert (o == 7.0).all() and (lse == 7.0).all()
    with pytest.raises(ea.AttnError):
        ea.attn_fwd_splitkv(q, k, v, 2, ws=torch.empty(16, dtype=torch.uint8, device="cuda"))
