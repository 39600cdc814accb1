"""Pins of the fp64 backward oracle (``oracle.backward``).

The gradients are pinned to the gradient the pages print for their worked example, to
central differences of the (separately pinned) forward oracle on tiny random problems,
and to invariants of the definition.  A slip in the backward (a dropped D term, a wrong
sign, a missing scale, a transposed operand, the causal mask left out) fails at least
one of them.  None of these tests touches the GPU library.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _grad_fixture():
    with open(os.path.join(GOLDEN, "score_gradient.json")) as f:
        return json.load(f)


def test_dk_of_the_worked_example_is_the_printed_score_gradient():
    """One query q = 1, keys k_j = s_j, values v_j, scale 1, dO = 1 (d = 1): then
    dK_j = dS_j * q = dy/ds_j, the central-difference gradient the page prints; dV_j is
    the probability p_j; dQ = sum_j dy/ds_j * s_j."""
    g = _grad_fixture()
    s = np.array(g["scores"])
    vals = np.array(g["values"])
    gp = np.array(g["dy_dscores"])
    tol = 0.5 * 10.0 ** -g["printed_decimals"] + 1e-9
    dq, dk, dv = oracle.attention_bwd(np.array([[1.0]]), s[:, None], vals[:, None],
                                      np.array([[1.0]]), 1.0)
    np.testing.assert_allclose(dk[:, 0], gp, atol=tol, rtol=0)
    assert abs(dk.sum()) < 1e-12
    y = float(oracle.attention(np.array([[1.0]]), s[:, None], vals[:, None], 1.0)[0][0, 0])
    np.testing.assert_allclose(dv[:, 0], gp / (vals - y), atol=2e-6, rtol=0)
    assert abs(dq[0, 0] - float(gp @ s)) <= tol * np.abs(s).sum()


def test_worked_example_embedded_in_a_head_keeps_the_printed_gradient():
    """The d = 64 embedding the GPU tests use (q = e0, k_j = s_j e0, v_j = value_j e0,
    dO = e0): column 0 carries the printed gradient, every other column is zero."""
    g = _grad_fixture()
    d = 64
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((4, d)); k[:, 0] = g["scores"]
    v = np.zeros((4, d)); v[:, 0] = g["values"]
    do = np.zeros((1, d)); do[0, 0] = 1.0
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 1.0)
    tol = 0.5 * 10.0 ** -g["printed_decimals"] + 1e-9
    np.testing.assert_allclose(dk[:, 0], g["dy_dscores"], atol=tol, rtol=0)
    assert np.abs(dk[:, 1:]).max() == 0.0 and np.abs(dv[:, 1:]).max() == 0.0
    assert np.abs(dq[:, 1:]).max() == 0.0


@pytest.mark.parametrize("shape,causal", [((2, 5, 7, 3), False), ((2, 5, 7, 3), True),
                                          ((1, 6, 4, 2), True), ((1, 3, 3, 4), False)])
def test_gradients_match_central_differences_of_the_forward(shape, causal):
    """L = sum(O * dO) with the forward oracle; every partial derivative of L by central
    differences equals the analytic gradient (Sq > Sk causal leaves rows fully masked)."""
    BH, Sq, Sk, d = shape
    rng = np.random.default_rng(11)
    q = rng.standard_normal((BH, Sq, d))
    k = rng.standard_normal((BH, Sk, d))
    v = rng.standard_normal((BH, Sk, d))
    do = rng.standard_normal((BH, Sq, d))
    scale = 0.7

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, scale, causal)
        return float(np.sum(o * do))

    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p = [xp if x is y else y for y in (q, k, v)]
            args_m = [xm if x is y else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, atol=2e-7, rtol=0)


def test_gradient_invariants():
    """Rows of dS sum to zero, so sum_j dK_j = 0; probabilities sum to one, so
    sum_j dV_j = sum_i dO_i over rows with visible keys; D equals sum(dO * O); the
    gradients are linear in dO; fully masked rows get dQ = 0."""
    rng = np.random.default_rng(5)
    BH, Sq, Sk, d = 3, 9, 6, 5
    q, do = rng.standard_normal((2, BH, Sq, d))
    k, v = rng.standard_normal((2, BH, Sk, d))
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.4, causal)
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
        o, lse = oracle.attention(q, k, v, 0.4, causal)
        live = np.isfinite(lse)
        np.testing.assert_allclose(dv.sum(axis=1), (do * live[..., None]).sum(axis=1), atol=1e-12)
        p = oracle.softmax_probs(q, k, 0.4, causal)
        dp = do @ np.swapaxes(v, -1, -2)
        np.testing.assert_allclose(oracle.row_dot(o, do), (p * dp).sum(-1), atol=1e-12)
        if causal:  # Sq - Sk = 3 rows see no key
            assert not live[:, :3].any() and live[:, 3:].all()
            assert np.abs(dq[:, :3]).max() == 0.0
        g2 = oracle.attention_bwd(q, k, v, 2.5 * do, 0.4, causal)
        for a, b in zip(g2, (dq, dk, dv)):
            np.testing.assert_allclose(a, 2.5 * b, atol=1e-12)
