"""Pins of the fp64 oracle against values the pages print, closed forms, invariants and
a 50-digit brute force on tiny inputs.

Each test is chosen so that a plausible slip in the oracle (a dropped scale, a sign, a
transposed operand, a wrong causal offset, a merge that forgets to rescale) fails at
least one of them.  None of these tests touches the GPU library.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _example():
    """Worked example as a single-query, d=1 attention problem with scale 1."""
    g = _load("worked_example.json")
    q = np.array([[1.0]])
    k = np.array(g["scores"])[:, None]
    v = np.array(g["values"])[:, None]
    return g, q, k, v


# --------------------------------------------------------------------------- printed values
def test_worked_example_full_softmax():
    g, q, k, v = _example()
    o, lse = oracle.attention(q, k, v, 1.0)
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    assert abs(o[0, 0] - g["merged_output"]) <= tol


def test_worked_example_two_block_states():
    g, q, k, v = _example()
    states = oracle.split_states(q, k, v, 1.0, 2)
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    for (m, l, u), want in zip(states, g["two_block_split"]):
        assert m[0] == want["m"]
        assert abs(l[0] - want["l"]) <= tol
        assert abs(u[0, 0] - want["u"]) <= tol
    o, _ = oracle.merge_states(states)
    assert abs(o[0, 0] - g["merged_output"]) <= tol


def test_worked_example_split_bounds_are_the_pages_blocks():
    g, _, _, _ = _example()
    bounds = oracle.split_bounds(4, 2)
    assert [list(range(a, b)) for a, b in bounds] == [b["keys"] for b in g["two_block_split"]]


def test_naive_average_reproduces_the_pages_counterexample_and_merge_does_not():
    g, q, k, v = _example()
    states = oracle.split_states(q, k, v, 1.0, 2)
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    bad = oracle.naive_average(states)
    assert abs(bad[0, 0] - g["naive_average_of_block_outputs"]) <= tol
    o, _ = oracle.merge_states(states)
    assert abs(o[0, 0] - g["naive_average_of_block_outputs"]) > 0.5


def test_score_gradient_matches_the_pages_central_difference():
    """Central difference of the oracle's output w.r.t. the four scores equals the
    gradient the page prints; this pins the softmax probabilities themselves."""
    g = _load("score_gradient.json")
    s0 = np.array(g["scores"], dtype=np.float64)
    v = np.array(g["values"])[:, None]
    q = np.array([[1.0]])

    def y(s):
        o, _ = oracle.attention(q, s[:, None], v, 1.0)
        return o[0, 0]

    h = 1e-5
    grad = np.array([(y(s0 + h * e) - y(s0 - h * e)) / (2 * h) for e in np.eye(4)])
    tol = 0.5 * 10.0 ** -g["printed_decimals"] + 1e-8
    np.testing.assert_allclose(grad, g["dy_dscores"], atol=tol, rtol=0)
    assert abs(grad.sum()) < 1e-9


def test_softmax_probs_agree_with_the_printed_gradient():
    """The printed gradient is p_j (v_j - y): recover p from it and compare."""
    g = _load("score_gradient.json")
    q = np.array([[1.0]])
    k = np.array(g["scores"])[:, None]
    v = np.array(g["values"])
    p = oracle.softmax_probs(q, k, 1.0)[0]
    y = float(p @ v)
    implied = np.array(g["dy_dscores"]) / (v - y)
    # printed to 6 decimals; |v - y| >= 0.61 bounds the amplification to < 1e-6
    np.testing.assert_allclose(p, implied, atol=2e-6, rtol=0)


# --------------------------------------------------------------------------- brute force
def _brute(q, k, v, scale, causal):
    """50-digit reference written as explicit loops (independent of NumPy)."""
    mpmath.mp.dps = 50
    Sq, d = q.shape
    Sk = k.shape[0]
    O = np.zeros((Sq, v.shape[1]))
    L = np.zeros(Sq)
    for i in range(Sq):
        s = []
        for j in range(Sk):
            if causal and j > i + (Sk - Sq):
                continue
            acc = mpmath.mpf(0)
            for t in range(d):
                acc += mpmath.mpf(float(q[i, t])) * mpmath.mpf(float(k[j, t]))
            s.append((j, mpmath.mpf(float(scale)) * acc))
        if not s:
            O[i, :] = 0.0
            L[i] = -math.inf
            continue
        z = mpmath.fsum(mpmath.exp(x) for _, x in s)
        for c in range(v.shape[1]):
            num = mpmath.fsum(mpmath.exp(x) * mpmath.mpf(float(v[j, c])) for j, x in s)
            O[i, c] = float(num / z)
        L[i] = float(mpmath.log(z))
    return O, L


@pytest.mark.parametrize("Sq,Sk,d,causal,scale", [
    (1, 1, 1, False, 1.0),
    (3, 5, 2, False, 0.37),
    (5, 3, 3, False, 1.9),
    (4, 4, 2, True, 0.5),
    (6, 3, 2, True, 1.3),     # Sq > Sk: the first 3 rows see no key at all
    (3, 7, 4, True, 0.8),     # Sq < Sk: bottom-right alignment
    (8, 8, 4, True, 2.5),
    (2, 6, 3, False, 40.0),   # very large scores: exercises the max shift
])
def test_brute_force_tiny_shapes(Sq, Sk, d, causal, scale):
    rng = np.random.default_rng(1000 + Sq * 100 + Sk * 10 + d)
    q = rng.standard_normal((Sq, d))
    k = rng.standard_normal((Sk, d))
    v = rng.standard_normal((Sk, 3))
    o, lse = oracle.attention(q, k, v, scale, causal)
    bo, bl = _brute(q, k, v, scale, causal)
    np.testing.assert_allclose(o, bo, atol=1e-12, rtol=1e-12)
    fin = np.isfinite(bl)
    np.testing.assert_array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], bl[fin], atol=1e-12, rtol=1e-13)
    for n in range(1, Sk + 3):  # more chunks than keys leaves several empty ones
        so, sl = oracle.attention_split(q, k, v, scale, n, causal)
        np.testing.assert_allclose(so, bo, atol=1e-12, rtol=1e-12)
        np.testing.assert_allclose(sl[fin], bl[fin], atol=1e-12, rtol=1e-13)
        assert np.all(np.isneginf(sl[~fin]))


# --------------------------------------------------------------------------- invariants
def test_split_counts_one_to_four_give_the_same_example_output():
    g, q, k, v = _example()
    ref_o, ref_l = oracle.attention(q, k, v, 1.0)
    for n in (1, 2, 3, 4):
        bounds = oracle.split_bounds(4, n)
        if n == 3:
            assert bounds[-1][0] == bounds[-1][1]  # the empty tail block
        o, lse = oracle.attention_split(q, k, v, 1.0, n)
        assert abs(o[0, 0] - ref_o[0, 0]) < 1e-14
        assert abs(lse[0] - ref_l[0]) < 1e-14


def test_empty_chunk_state_is_neutral():
    g, q, k, v = _example()
    m, l, u = oracle.partial_state(q, k, v, 1.0, 4, 4)
    assert np.isneginf(m[0]) and l[0] == 0.0 and np.all(u == 0.0)


def test_probabilities_sum_to_one():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 3, 17, 8))
    k = rng.standard_normal((2, 3, 23, 8))
    for causal in (False, True):
        p = oracle.softmax_probs(q, k, 0.35, causal)
        np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
        assert np.all(p >= 0)


def test_key_permutation_invariance_non_causal():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 2, 9, 16))
    k = rng.standard_normal((1, 2, 31, 16))
    v = rng.standard_normal((1, 2, 31, 16))
    perm = rng.permutation(31)
    o1, l1 = oracle.attention(q, k, v, 0.25)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.25)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_single_key_returns_that_value():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 4))
    k = rng.standard_normal((1, 4))
    v = rng.standard_normal((1, 6))
    o, lse = oracle.attention(q, k, v, 0.7)
    np.testing.assert_allclose(o, np.repeat(v, 5, axis=0), atol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * (q @ k[0]), atol=1e-14)


def test_zero_query_gives_mean_of_values_and_log_sk():
    rng = np.random.default_rng(10)
    k = rng.standard_normal((13, 4))
    v = rng.standard_normal((13, 5))
    o, lse = oracle.attention(np.zeros((2, 4)), k, v, 1.0)
    np.testing.assert_allclose(o, np.tile(v.mean(0), (2, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(13), atol=1e-14)


def test_causal_first_row_sees_only_the_first_key():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((6, 4))
    k = rng.standard_normal((6, 4))
    v = rng.standard_normal((6, 3))
    o, lse = oracle.attention(q, k, v, 0.9, causal=True)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    assert abs(lse[0] - 0.9 * q[0] @ k[0]) < 1e-14


def test_causal_row_equals_non_causal_over_its_visible_prefix():
    rng = np.random.default_rng(12)
    for Sq, Sk in ((7, 7), (4, 9), (9, 4)):
        q = rng.standard_normal((Sq, 5))
        k = rng.standard_normal((Sk, 5))
        v = rng.standard_normal((Sk, 5))
        o, lse = oracle.attention(q, k, v, 0.6, causal=True)
        for i in range(Sq):
            last = i + Sk - Sq
            if last < 0:
                assert np.all(o[i] == 0) and np.isneginf(lse[i])
                continue
            oi, li = oracle.attention(q[i:i + 1], k[:last + 1], v[:last + 1], 0.6)
            np.testing.assert_allclose(o[i], oi[0], atol=1e-14)
            assert abs(lse[i] - li[0]) < 1e-13


def test_equal_maxima_average_the_tied_values():
    q = np.array([[1.0]])
    k = np.array([[3.0], [3.0], [-50.0]])
    v = np.array([[2.0], [6.0], [100.0]])
    o, lse = oracle.attention(q, k, v, 1.0)
    assert abs(o[0, 0] - 4.0) < 1e-15
    assert abs(lse[0] - (3.0 + math.log(2.0 + math.exp(-53.0)))) < 1e-14


def test_large_scale_tends_to_hardmax():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((16, 8))
    v = rng.standard_normal((16, 3))
    o, _ = oracle.attention(q, k, v, 1e4)
    np.testing.assert_allclose(o, v[np.argmax(q @ k.T, axis=1)], atol=1e-12)


def test_mask_shapes():
    m = oracle.visible_mask(3, 5, True)
    assert m.tolist() == [[True, True, True, False, False],
                          [True, True, True, True, False],
                          [True, True, True, True, True]]
    m = oracle.visible_mask(5, 3, True)
    assert m.sum(axis=1).tolist() == [0, 0, 1, 2, 3]
    assert oracle.visible_mask(4, 4, False).all()


def test_flop_count_convention():
    assert oracle.flops(1, 8, 8192, 8192, 128, False) == 4 * 8 * 8192 ** 2 * 128
    assert oracle.flops(1, 8, 8192, 8192, 128, True) == 2 * 8 * 8192 ** 2 * 128


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 16])
def test_split_invariance_random_batches(n):
    rng = np.random.default_rng(20 + n)
    q = rng.standard_normal((2, 2, 5, 8))
    k = rng.standard_normal((2, 2, 37, 8))
    v = rng.standard_normal((2, 2, 37, 8))
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.3, causal)
        so, sl = oracle.attention_split(q, k, v, 0.3, n, causal)
        np.testing.assert_allclose(so, o, atol=1e-13)
        np.testing.assert_allclose(sl, lse, atol=1e-13)


def test_row_sample_matches_full_problem():
    rng = np.random.default_rng(30)
    q = rng.standard_normal((1, 1, 40, 8))
    k = rng.standard_normal((1, 1, 50, 8))
    v = rng.standard_normal((1, 1, 50, 8))
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.4, causal)
        so, sl = oracle.attention(q[:, :, rows], k, v, 0.4, causal, Sq_total=40, q_index=rows)
        np.testing.assert_allclose(so, o[:, :, rows], atol=1e-14)
        np.testing.assert_allclose(sl, lse[:, :, rows], atol=1e-14)
