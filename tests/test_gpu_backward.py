"""GPU parity of the backward (attn_bwd through the C ABI) against the fp64 oracle.

Tolerance, derived from the arithmetic the kernels perform (elementwise, per output):
the library rounds dO, P and dS to bf16 (unit roundoff u = 2^-8) as MFMA operands and
accumulates in fp32 (n terms: about n * 2^-24 of the sum of magnitudes).  Propagating
those roundings through dP = dO V^T, D = rowsum(dO * O), dS = P (dP - D) and the three
products gives a first-order bound for every element of dQ, dK and dV, computed below
from the oracle's own fp64 P, dP and dS; the GPU must stay within twice that bound
(the factor covers second-order terms).  Inputs whose scores are large (rows of Q
scaled by 30) get a proportionally larger bound, as the arithmetic says they should:
dK = scale dS^T Q multiplies the bf16 rounding of dS by |Q|.

The worked example of the pages is checked against its printed score gradient (dK of
the embedded problem), and the whole forward-then-backward chain against the oracle.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_helpers import to_device, upload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import exact_attention_82_amd as ea

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits)
U_F32 = 2.0 ** -24


def _np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


def _inputs(B, H, Sq, Sk, d, seed, hot=0.0):
    inp = si.make_attention_inputs(B, H, Sq, Sk, d, seed=seed, dtype="bf16", hot_row_frac=hot)
    rng = np.random.default_rng(seed + 1000)
    do = rng.standard_normal((B, H, Sq, d), dtype=np.float32)
    return inp, do


def _bound(q, k, v, o, do, scale, causal, extra_d=0.0, extra_lse=0.0):
    """Elementwise first-order error bounds (dQ, dK, dV) of the bf16 / fp32 arithmetic for
    one head (fp64 arrays [S, d]); extra_d / extra_lse add an error already present in
    the O / lse handed to the backward."""
    Sq, d = q.shape
    Sk = k.shape[0]
    p = oracle.softmax_probs(q, k, scale, causal)
    dp = do @ v.T
    dsum = (p * dp).sum(-1)
    ds = p * (dp - dsum[:, None])
    aq, ak, av, ado = np.abs(q), np.abs(k), np.abs(v), np.abs(do)
    e_s = scale * d * U_F32 * (aq @ ak.T)                    # fp32 score accumulation
    e_p = p * (e_s * np.log(2.0) + 2.0 ** -21 + extra_lse)   # exp2 of the shifted score
    e_dp = (U_BF16 + d * U_F32) * (ado @ av.T)               # bf16 dO, fp32 accumulation
    e_d = d * U_F32 * (ado * np.abs(o)).sum(-1) + extra_d * ado.sum(-1)
    e_ds = e_p * np.abs(dp - dsum[:, None]) + p * (e_dp + e_d[:, None])
    e_dsb = e_ds + U_BF16 * np.abs(ds)                      # dS rounded to bf16
    e_dv = (e_p + 2 * U_BF16 * p).T @ ado + Sq * U_F32 * (p.T @ ado)
    e_dk = scale * (e_dsb.T @ aq) + Sq * U_F32 * scale * (np.abs(ds).T @ aq)
    e_dq = scale * (e_dsb @ ak) + Sk * U_F32 * scale * (np.abs(ds) @ ak)
    return e_dq, e_dk, e_dv


def _run_bwd(q, k, v, o, lse, do, scale, causal):
    dev = "cuda"
    ot = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float32)).to(dev)
    lt = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to(dev)
    dt = torch.from_numpy(np.ascontiguousarray(do, dtype=np.float32)).to(dev)
    dq, dk, dv = ea.attn_bwd(q, k, v, ot, lt, dt, scale=scale, causal=causal)
    return _np(dq), _np(dk), _np(dv)


def _check_heads(inp, do, scale, causal, got, extra_d=0.0, extra_lse=0.0, label=""):
    B, H, Sq, Sk, d = inp.B, inp.H, inp.Sq, inp.Sk, inp.d
    q = inp.q64.reshape(B * H, Sq, d)
    k = inp.k64.reshape(B * H, Sk, d)
    v = inp.v64.reshape(B * H, Sk, d)
    dof = do.reshape(B * H, Sq, d).astype(np.float64)
    gq, gk, gv = (x.reshape(B * H, -1, d) for x in got)
    worst = 0.0
    for h in range(B * H):
        o, _ = oracle.attention(q[h], k[h], v[h], scale, causal)
        ref = oracle.attention_bwd(q[h], k[h], v[h], dof[h], scale, causal)
        bnd = _bound(q[h], k[h], v[h], o, dof[h], scale, causal, extra_d, extra_lse)
        for name, g_, r_, b_ in zip(("dQ", "dK", "dV"), (gq[h], gk[h], gv[h]), ref, bnd):
            err = np.abs(g_ - r_)
            lim = 2.0 * b_ + 1e-7
            bad = err > lim
            worst = max(worst, float((err / lim).max()))
            assert not bad.any(), (
                f"{label} head {h} {name}: {int(bad.sum())} elements over the bound; "
                f"max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}, "
                f"bound there {lim.flat[err.argmax()]:.3e}, max|ref| {np.abs(r_).max():.3e}")
    print(f"{label}: max err / bound = {worst:.3f}", flush=True)
    return worst


def _oracle_fwd(inp, scale, causal):
    B, H, Sq, Sk, d = inp.B, inp.H, inp.Sq, inp.Sk, inp.d
    o, lse = oracle.attention(inp.q64.reshape(B * H, Sq, d), inp.k64.reshape(B * H, Sk, d),
                              inp.v64.reshape(B * H, Sk, d), scale, causal)
    return o.reshape(B, H, Sq, d), lse.reshape(B, H, Sq)


@pytest.mark.parametrize("B,H,Sq,Sk,d,causal,hot", [
    (1, 2, 300, 300, 64, False, 0.0),
    (1, 2, 300, 300, 64, True, 0.0),
    (2, 3, 257, 190, 128, False, 0.0),
    (2, 3, 257, 190, 128, True, 0.0),     # Sq > Sk: the first 67 rows see no key
    (1, 2, 190, 333, 128, True, 0.0),     # Sq < Sk: bottom-right alignment
    (1, 2, 700, 700, 128, True, 0.01),    # 1 % of query rows scaled by 30
    (1, 1, 1000, 1000, 128, False, 0.0),
    (1, 1, 1, 5, 64, False, 0.0),
    (1, 1, 33, 1, 128, True, 0.0),
    (1, 2, 300, 300, 256, False, 0.0),
    (2, 1, 257, 190, 256, True, 0.0),
])
def test_backward_matches_oracle(B, H, Sq, Sk, d, causal, hot):
    inp, do = _inputs(B, H, Sq, Sk, d, seed=31 + Sq + d, hot=hot)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _oracle_fwd(inp, scale, causal)
    q, k, v = upload(inp)
    got = _run_bwd(q, k, v, o, lse, do, scale, causal)
    _check_heads(inp, do, scale, causal, got, label=f"bwd {B}x{H}x{Sq}x{Sk} d={d} causal={causal}")
    if causal and Sq > Sk:  # rows with no visible key: no gradient reaches Q
        assert np.abs(got[0].reshape(B, H, Sq, d)[:, :, : Sq - Sk]).max() == 0.0


def test_backward_worked_example_gives_the_printed_score_gradient():
    """Embedded worked example (q = e0, k_j = s_j e0, v_j = value_j e0, scale 1, dO = e0):
    dK[:, 0] is the page's central-difference score gradient, up to the bf16 rounding
    of dS (2^-8 relative)."""
    with open(os.path.join(GOLDEN, "score_gradient.json")) as f:
        g = json.load(f)
    d = 64
    inp = si.worked_example_inputs(d, "bf16")
    do = np.zeros((1, 1, 1, d), dtype=np.float32)
    do[0, 0, 0, 0] = 1.0
    o, lse = _oracle_fwd(inp, 1.0, False)
    q, k, v = upload(inp)
    dq, dk, dv = _run_bwd(q, k, v, o, lse, do, 1.0, False)
    gp = np.array(g["dy_dscores"])
    np.testing.assert_allclose(dk[0, 0, :, 0], gp, rtol=2 * U_BF16, atol=1e-6)
    assert np.abs(dk[0, 0, :, 1:]).max() == 0.0 and np.abs(dq[0, 0, :, 1:]).max() == 0.0
    # dQ = sum_j bf16(dS_j) s_j: each rounding (2^-8 relative) is multiplied by s_j
    sc = np.array(g["scores"])
    tol = U_BF16 * float(np.abs(gp * sc).sum()) + 1e-6
    np.testing.assert_allclose(dq[0, 0, 0, 0], float(gp @ sc), rtol=0, atol=tol)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_then_backward_chain(causal):
    """O and lse from attn_fwd feed attn_bwd directly; the forward's own error enters D
    and P and is added to the bound."""
    B, H, S, d = 1, 2, 520, 128
    inp, do = _inputs(B, H, S, S, d, seed=77)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q, k, v = upload(inp)
    o_t, l_t = ea.attn_fwd(q, k, v, scale=scale, causal=causal)
    o_ref, l_ref = _oracle_fwd(inp, scale, causal)
    eo = float(np.abs(_np(o_t) - o_ref).max())
    el = float(np.abs(_np(l_t) - l_ref).max())
    dt = torch.from_numpy(do).cuda()
    dq, dk, dv = ea.attn_bwd(q, k, v, o_t, l_t, dt, scale=scale, causal=causal)
    _check_heads(inp, do, scale, causal, (_np(dq), _np(dk), _np(dv)), extra_d=eo, extra_lse=el,
                 label=f"fwd+bwd causal={causal} (fwd err O {eo:.1e}, lse {el:.1e})")


def test_backward_is_deterministic_and_leaves_inputs_alone():
    B, H, S, d = 2, 2, 384, 128
    inp, do = _inputs(B, H, S, S, d, seed=5)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _oracle_fwd(inp, scale, True)
    q, k, v = upload(inp)
    first = _run_bwd(q, k, v, o, lse, do, scale, True)
    second = _run_bwd(q, k, v, o, lse, do, scale, True)
    for a, b in zip(first, second):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_d256_long_sweeps(causal):
    """d = 256 at S = 1024 (32 query tiles per key sweep, 8 key tiles per query sweep): the
    dK/dV and dQ accumulators of these kernels run through many MFMA chains per call."""
    B, H, S, d = 1, 2, 1024, 256
    inp, do = _inputs(B, H, S, S, d, seed=77 + int(causal))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o, lse = _oracle_fwd(inp, scale, causal)
    q, k, v = upload(inp)
    got = _run_bwd(q, k, v, o, lse, do, scale, causal)
    _check_heads(inp, do, scale, causal, got, label=f"bwd 1x2x1024 d=256 causal={causal}")


def test_backward_one_head_at_training_size():
    """B=1, H=4, S=2048, d=128, causal: head 3 compared in full (the others must be finite)."""
    B, H, S, d = 1, 4, 2048, 128
    inp, do = _inputs(B, H, S, S, d, seed=9)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q, k, v = upload(inp)
    o_t, l_t = ea.attn_fwd(q, k, v, scale=scale, causal=True)
    dt = torch.from_numpy(do).cuda()
    dq, dk, dv = (_np(x) for x in ea.attn_bwd(q, k, v, o_t, l_t, dt, scale=scale, causal=True))
    assert all(np.isfinite(x).all() for x in (dq, dk, dv))
    o_ref, l_ref = _oracle_fwd(inp, scale, True)
    eo = float(np.abs(_np(o_t) - o_ref).max())
    el = float(np.abs(_np(l_t) - l_ref).max())
    h = 3
    one = si.AttentionInputs("bf16", 1, 1, S, S, d, 9, None, None, None,
                             inp.q64[:, h:h + 1], inp.k64[:, h:h + 1], inp.v64[:, h:h + 1])
    _check_heads(one, do[:, h:h + 1], scale, True,
                 (dq[:, h:h + 1], dk[:, h:h + 1], dv[:, h:h + 1]), extra_d=eo, extra_lse=el,
                 label="bwd 1x4x2048 d=128 causal, head 3")


def test_backward_split_sweeps_at_sixteen_heads():
    """B=1, H=16, S=2048, d=128, causal: the dK/dV and dQ grids (256 workgroups each) are
    resident at once, so the long key and query sweeps run in two halves, and the dK/dV
    halves (16 heads x 11 long key tiles) are added by the last workgroups of the dQ launch
    in more than one round per thread.  Heads 0 and 15 compared in full."""
    B, H, S, d = 1, 16, 2048, 128
    inp, do = _inputs(B, H, S, S, d, seed=12)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q, k, v = upload(inp)
    o_t, l_t = ea.attn_fwd(q, k, v, scale=scale, causal=True)
    dt = torch.from_numpy(do).cuda()
    dq, dk, dv = (_np(x) for x in ea.attn_bwd(q, k, v, o_t, l_t, dt, scale=scale, causal=True))
    assert all(np.isfinite(x).all() for x in (dq, dk, dv))
    o_ref, l_ref = _oracle_fwd(inp, scale, True)
    eo = float(np.abs(_np(o_t) - o_ref).max())
    el = float(np.abs(_np(l_t) - l_ref).max())
    for h in (0, H - 1):
        one = si.AttentionInputs("bf16", 1, 1, S, S, d, 12, None, None, None,
                                 inp.q64[:, h:h + 1], inp.k64[:, h:h + 1], inp.v64[:, h:h + 1])
        _check_heads(one, do[:, h:h + 1], scale, True,
                     (dq[:, h:h + 1], dk[:, h:h + 1], dv[:, h:h + 1]), extra_d=eo, extra_lse=el,
                     label=f"bwd 1x16x2048 d=128 causal, head {h}")


def test_backward_refuses_what_it_does_not_support():
    inp, do = _inputs(1, 1, 64, 64, 64, seed=1)
    q, k, v = upload(inp)
    o = torch.zeros(1, 1, 64, 64, device="cuda")
    l = torch.zeros(1, 1, 64, device="cuda")
    dt = torch.from_numpy(do).cuda()
    with pytest.raises(ea.AttnError):
        ea.attn_bwd(q.float(), k.float(), v.float(), o, l, dt)    # fp32: not supported
    with pytest.raises(ea.AttnError):
        ea.attn_bwd(q, k, v, o, l, dt, ws=torch.empty(16, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_at_the_c2_shape_two_heads(causal):
    """B=8, H=32, S=2048, d=64 (the c2 workload's shape): the first and the last head
    compared in full against the oracle (the others must be finite)."""
    B, H, S, d = 8, 32, 2048, 64
    inp, do = _inputs(B, H, S, S, d, seed=2)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q, k, v = upload(inp)
    o_t, l_t = ea.attn_fwd(q, k, v, scale=scale, causal=causal)
    dt = torch.from_numpy(do).cuda()
    grads = [_np(x) for x in ea.attn_bwd(q, k, v, o_t, l_t, dt, scale=scale, causal=causal)]
    assert all(np.isfinite(x).all() for x in grads)
    o_all, l_all = _np(o_t), _np(l_t)
    for (b, h) in ((0, 0), (B - 1, H - 1)):
        qh, kh, vh = (x[b, h] for x in (inp.q64, inp.k64, inp.v64))
        o_ref, l_ref = oracle.attention(qh, kh, vh, scale, causal)
        eo = float(np.abs(o_all[b, h] - o_ref).max())
        el = float(np.abs(l_all[b, h] - l_ref).max())
        one = si.AttentionInputs("bf16", 1, 1, S, S, d, 2, None, None, None,
                                 qh[None, None], kh[None, None], vh[None, None])
        _check_heads(one, do[b:b + 1, h:h + 1], scale, causal,
                     tuple(x[b:b + 1, h:h + 1] for x in grads), extra_d=eo, extra_lse=el,
                     label=f"bwd c2 shape head ({b},{h}) causal={causal}")
