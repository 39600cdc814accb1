"""Pins of the ragged-batch oracle (oracle.attention_varlen), CPU only.

The oracle applies the plain definition to each sequence's slices.  These tests pin it
to things that do not share that code path: a 50-digit brute force over the *packed*
rows with the visibility rule written on absolute row indices (which key rows belong
to the query row's sequence, and the causal rule relative to that sequence's corner),
the dense batched oracle when every sequence has the same length, and invariants
(a sequence's output ignores every other sequence; empty sequences).
"""
import math

import mpmath
import numpy as np
import pytest

import oracle


def _brute_packed(q, k, v, cu_q, cu_k, scale, causal):
    """50-digit loops over packed rows: key row j is visible to query row i iff j lies in
    the key range of i's sequence and, causal, (j - k0) <= (i - q0) + (nk - nq)."""
    mpmath.mp.dps = 50
    H, Tq, d = q.shape
    O = np.full((H, Tq, v.shape[2]), np.nan)
    L = np.full((H, Tq), np.nan)
    nb = len(cu_q) - 1
    for h in range(H):
        for i in range(Tq):
            owner = [b for b in range(nb) if cu_q[b] <= i < cu_q[b + 1]]
            if not owner:
                continue
            b = owner[0]
            q0, k0 = cu_q[b], cu_k[b]
            nq, nk = cu_q[b + 1] - q0, cu_k[b + 1] - k0
            s = []
            for j in range(k.shape[1]):
                if not (k0 <= j < k0 + nk):
                    continue
                if causal and (j - k0) > (i - q0) + (nk - nq):
                    continue
                acc = mpmath.fsum(mpmath.mpf(float(q[h, i, t])) * mpmath.mpf(float(k[h, j, t]))
                                  for t in range(d))
                s.append((j, mpmath.mpf(float(scale)) * acc))
            if not s:
                O[h, i] = 0.0
                L[h, i] = -math.inf
                continue
            z = mpmath.fsum(mpmath.exp(x) for _, x in s)
            for c in range(v.shape[2]):
                O[h, i, c] = float(mpmath.fsum(mpmath.exp(x) * mpmath.mpf(float(v[h, j, c]))
                                               for j, x in s) / z)
            L[h, i] = float(mpmath.log(z))
    return O, L


@pytest.mark.parametrize("lens_q,lens_k,causal", [
    ([3, 1, 4], [3, 1, 4], False),
    ([3, 1, 4], [3, 1, 4], True),
    ([2, 5, 3], [4, 2, 3], True),   # Sq != Sk per sequence: own bottom-right corners
    ([2, 0, 3], [1, 3, 0], True),   # an empty query range, and a sequence with no keys
    ([4, 2], [6, 5], False),
])
def test_varlen_oracle_matches_packed_brute_force(lens_q, lens_k, causal):
    rng = np.random.default_rng(7)
    H, d = 2, 3
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    q = rng.standard_normal((H, cu_q[-1], d))
    k = rng.standard_normal((H, cu_k[-1], d))
    v = rng.standard_normal((H, cu_k[-1], d))
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.7, causal)
    bo, bl = _brute_packed(q, k, v, cu_q, cu_k, 0.7, causal)
    np.testing.assert_allclose(o, bo, atol=1e-12, rtol=0)
    assert np.array_equal(np.isneginf(lse), np.isneginf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], atol=1e-12, rtol=0)


def test_equal_lengths_match_the_dense_batched_oracle():
    rng = np.random.default_rng(8)
    B, H, S, d = 3, 2, 5, 4
    q, k, v = (rng.standard_normal((B, H, S, d)) for _ in range(3))
    cu = np.arange(B + 1) * S
    pack = lambda t: np.ascontiguousarray(t.transpose(1, 0, 2, 3).reshape(H, B * S, d))
    for causal in (False, True):
        o, lse = oracle.attention_varlen(pack(q), pack(k), pack(v), cu, cu, 0.5, causal)
        ro, rl = oracle.attention(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, pack(ro), atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse, rl.transpose(1, 0, 2).reshape(H, B * S), atol=1e-13, rtol=0)


def test_sequences_do_not_see_each_other_and_gaps_stay_unwritten():
    rng = np.random.default_rng(9)
    H, d = 2, 4
    cu_q = np.array([0, 3, 7])
    cu_k = np.array([0, 5, 9])
    q = rng.standard_normal((H, 9, d))   # rows 7, 8 belong to no sequence
    k = rng.standard_normal((H, 9, d))
    v = rng.standard_normal((H, 9, d))
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.5, True)
    k2, v2 = k.copy(), v.copy()
    k2[:, 5:] += 3.0                      # perturb the second sequence's keys only
    v2[:, 5:] -= 2.0
    o2, lse2 = oracle.attention_varlen(q, k2, v2, cu_q, cu_k, 0.5, True)
    np.testing.assert_array_equal(o[:, :3], o2[:, :3])
    np.testing.assert_array_equal(lse[:, :3], lse2[:, :3])
    assert not np.allclose(o[:, 3:7], o2[:, 3:7])
    assert np.isnan(o[:, 7:]).all() and np.isnan(lse[:, 7:]).all()
