"""GPU parity of attn_fwd_varlen (ragged batches, packed head-major) against the fp64
oracle's per-sequence definition (oracle.attention_varlen), through the C ABI.

Length mixes cover empty sequences, one-row sequences, lengths on and off the 128-row
tile and the key-tile size, per-sequence Sq != Sk (causal alignment to each sequence's
own corner, fully masked rows), all three input types and head dims, rows no sequence
covers (must stay unwritten), and offsets that break the documented contract (clamped
on the device: the call must stay inside the buffers).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_helpers import check, scale_for, to_device

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import exact_attention_82_amd as ea

SENTINEL = 7.0


def _np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def _run(inp, cu_q, cu_k, causal, max_q=None, max_k=None, total_q=None):
    """attn_fwd_varlen on packed inputs; O and lse pre-filled with a sentinel."""
    q, k, v = (to_device(t[0], inp.dtype) for t in (inp.q, inp.k, inp.v))
    H, Tq, d = q.shape
    sq, sk, sv = inp.scales
    scale = scale_for(d)
    eff = float(np.float32(scale * sq * sk)) if inp.dtype == "fp8" else scale
    o = torch.full((H, Tq, d), SENTINEL, dtype=torch.float32, device="cuda")
    lse = torch.full((H, Tq), SENTINEL, dtype=torch.float32, device="cuda")
    lq, lk = np.diff(cu_q), np.diff(cu_k)
    mq = max_q if max_q is not None else max(1, int(lq.max()))
    mk = max_k if max_k is not None else max(1, int(lk.max()))
    ea.attn_fwd_varlen(q, k, v, torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(),
                       mq, mk, scale=eff, causal=causal, out=o, lse=lse)
    o, lse = _np(o), _np(lse)
    if inp.dtype == "fp8":
        covered = o != SENTINEL
        o = np.where(covered, o * np.float32(sv), o)
    return o, lse, scale


def _ref(inp, cu_q, cu_k, scale, causal):
    return oracle.attention_varlen(inp.q64[0], inp.k64[0], inp.v64[0], cu_q, cu_k, scale, causal)


CASES = [
    # dtype, d, query lengths, key lengths
    ("bf16", 128, [1, 127, 128, 129, 300, 0, 1000], [1, 127, 128, 129, 300, 0, 1000]),
    ("bf16", 64, [513, 77, 256, 1, 40], [400, 77, 900, 5, 0]),
    ("bf16", 256, [200, 130, 33], [200, 130, 257]),
    ("f32", 64, [33, 128, 70], [40, 128, 70]),
    ("f32", 128, [5, 190], [300, 64]),
    ("fp8", 128, [128, 64, 3], [2048, 999, 17]),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,lens_q,lens_k", CASES)
def test_varlen_matches_per_sequence_oracle(dtype, d, lens_q, lens_k, causal):
    inp, cu_q, cu_k = si.make_varlen_inputs(lens_q, lens_k, 2, d, seed=11, dtype=dtype)
    print(f"varlen {dtype} d={d} q={lens_q} k={lens_k} causal={causal}", flush=True)
    o, lse, scale = _run(inp, cu_q, cu_k, causal)
    ro, rl = _ref(inp, cu_q, cu_k, scale, causal)
    rows = ~np.isnan(rl[0])
    check(f"varlen {dtype} d={d} causal={causal}", o[:, rows], lse[:, rows], ro[:, rows],
          rl[:, rows], dtype)


def test_varlen_leaves_uncovered_rows_and_empty_sequences_alone():
    # rows 250..299 of Q belong to no sequence; sequence 1 has no keys (O = 0, lse = -inf)
    inp, _, _ = si.make_varlen_inputs([300], [200], 2, 128, seed=12, dtype="bf16")
    cu_q = np.array([0, 100, 250], dtype=np.int32)
    cu_k = np.array([0, 200, 200], dtype=np.int32)
    o, lse, scale = _run(inp, cu_q, cu_k, True)
    assert np.all(o[:, 250:] == SENTINEL) and np.all(lse[:, 250:] == SENTINEL)
    assert np.all(o[:, 100:250] == 0.0) and np.all(np.isneginf(lse[:, 100:250]))
    ro, rl = _ref(inp, cu_q, cu_k, scale, True)
    check("varlen gap", o[:, :100], lse[:, :100], ro[:, :100], rl[:, :100], "bf16")


def test_varlen_equal_lengths_equal_the_dense_call():
    # 4 * 16 * 5 = 320 workgroups: more than one per CU, so the dense call also takes the
    # plain kernel (small grids use the two-group kernel, which sums in another order)
    B, H, S, d = 4, 16, 640, 64
    inp = si.make_attention_inputs(B, H, S, S, d, seed=13, dtype="bf16")
    pack = lambda t: np.ascontiguousarray(t.transpose(1, 0, 2, 3).reshape(H, B * S, d))
    q, k, v = (to_device(pack(t), "bf16") for t in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(si.cu_seqlens([S] * B)).cuda()
    scale = scale_for(d)
    o, lse = ea.attn_fwd_varlen(q, k, v, cu, cu, S, S, scale=scale, causal=False)
    qd, kd, vd = (to_device(t, "bf16") for t in (inp.q, inp.k, inp.v))
    od, ld = ea.attn_fwd(qd, kd, vd, scale=scale, causal=False)
    od = _np(od).transpose(1, 0, 2, 3).reshape(H, B * S, d)
    ld = _np(ld).transpose(1, 0, 2).reshape(H, B * S)
    # the same kernel instance on the same rows: identical bits
    np.testing.assert_array_equal(_np(o), od)
    np.testing.assert_array_equal(_np(lse), ld)


def test_varlen_offsets_outside_the_contract_stay_in_bounds():
    # decreasing offsets, offsets past total and lengths past max_seqlen: the device
    # clamps them, so the call completes and writes only finite values or nothing
    inp, _, _ = si.make_varlen_inputs([200], [300], 2, 128, seed=14, dtype="bf16")
    cu_q = np.array([0, 50, 30, 400], dtype=np.int32)
    cu_k = np.array([0, 500, 100, 50], dtype=np.int32)
    o, lse, _ = _run(inp, cu_q, cu_k, False, max_q=256, max_k=256)
    assert np.all(np.isfinite(o))
    assert not np.any(np.isnan(lse))


def test_varlen_length_mix_at_scale_sampled_rows():
    # 12 sequences of 1..4096 tokens, H=8, d=128, bf16: every sequence's first, last and
    # tile-edge rows plus random rows of two heads against the oracle evaluated row by row
    lens = si.varlen_lengths(12, 1, 4096, seed=15)
    inp, cu_q, cu_k = si.make_varlen_inputs(lens, lens, 8, 128, seed=16, dtype="bf16")
    rng = np.random.default_rng(17)
    for causal in (False, True):
        o, lse, scale = _run(inp, cu_q, cu_k, causal)
        for h in (0, 5):
            for b in range(len(lens)):
                a, n = int(cu_q[b]), int(lens[b])
                rows = {0, n - 1, min(n - 1, 127), min(n - 1, 128)} | set(rng.integers(0, n, size=6).tolist())
                rows = np.array(sorted(rows), dtype=np.int64)
                qk = slice(int(cu_k[b]), int(cu_k[b + 1]))
                ro, rl = oracle.attention(inp.q64[0, h, a + rows], inp.k64[0, h, qk], inp.v64[0, h, qk],
                                          scale, causal, Sq_total=n, q_index=rows)
                check(f"varlen mix causal={causal} h={h} b={b}", o[h, a + rows][None], lse[h, a + rows][None],
                      ro[None], rl[None], "bf16")
