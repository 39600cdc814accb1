"""Plain fp64 CPU reference for the gradients of exact attention (backward).

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: nothing in the product path may
import or call it, and it shares no code with the HIP library.

For one (batch, head), with P = softmax(S) the attention probabilities of the forward
(S = scale * Q K^T, masked entries -inf, fully masked rows P = 0) and O = P V, the
gradients of a scalar loss L with upstream gradient dO = dL/dO are the chain rule of that
definition, written out and materialised:

    dV  = P^T dO
    dP  = dO V^T
    D_i = sum_j P_ij dP_ij            (= sum_d dO_id O_id)
    dS  = P * (dP - D)                (elementwise; 0 where masked)
    dQ  = scale * dS K
    dK  = scale * dS^T Q

The "FlashAttention_02" page, section "Training and deployment: backward consistency of
split and reduction", states the key fact behind dS: the derivative of the output with
respect to a score depends on the *global* output y (for one query and a scalar output,
dy/ds_j = p_j (v_j - y), which is dS with dP_j = v_j and D = y), and it prints that
gradient for its worked example; the same section notes that dK and dV accumulate across
queries, the other direction from the forward's split.
"""
from __future__ import annotations

import numpy as np

from .attention import softmax_probs

__all__ = ["attention_bwd", "row_dot"]


def row_dot(o, do):
    """D_i = sum_d dO_id O_id, the per-row term of dS, from the forward output."""
    return np.sum(np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64), axis=-1)


def attention_bwd(q, k, v, do, scale, causal=False):
    """Gradients (dQ, dK, dV) of L with dL/dO = ``do`` for O = attention(q, k, v).

    Shapes [..., Sq, d] for q and do, [..., Sk, d] for k and v; float64 results.  The
    causal mask is the forward's (key j hidden from query i when j > i + Sk - Sq).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    p = softmax_probs(q, k, scale, causal)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    dsum = np.sum(p * dp, axis=-1)
    ds = p * (dp - dsum[..., None])
    dq = np.float64(scale) * np.matmul(ds, k)
    dk = np.float64(scale) * np.matmul(np.swapaxes(ds, -1, -2), q)
    return dq, dk, dv
