"""Plain fp64 CPU reference for exact scaled-dot-product attention (forward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library: no kernels, no headers, no constants, no helpers.

What it computes is the plain definition, written out and fully materialised:

    S = scale * Q K^T            (Sq x Sk per (batch, head))
    S_ij = -inf  where masked    (causal: key j is hidden from query i when j > i + Sk - Sq)
    m_i  = max_j S_ij
    P    = exp(S - m),  l_i = sum_j P_ij
    O    = (P V) / l,   lse_i = m_i + ln l_i

("FlashAttention_02" page, sections 3.1 and 4.1: FA2 computes the same exact dense
attention; "Inside FlashAttention-3" page, section 2: the two-level online softmax
reaches exactly this result.)  Rows whose every key is masked have no softmax; this
reference returns O = 0 and lse = -inf for them (log of an empty sum).

The split-K functions follow the split-K section of the "FlashAttention_02" page: the
keys are cut into chunks, each chunk keeps its local (m, l, u) with u the
*unnormalised* weighted value sum, and the merge rescales every chunk by
exp(m_s - M) against the global maximum M before summing and normalising once.

Inputs are float64 arrays holding the exact values the GPU receives (bf16 / E4M3 values
already rounded and, for fp8, multiplied by their per-tensor scale).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visible_mask", "scores", "softmax_probs", "attention", "split_bounds",
    "partial_state", "split_states", "merge_states", "naive_average", "attention_split",
    "attention_varlen",
]


def visible_mask(Sq: int, Sk: int, causal: bool, q_index=None) -> np.ndarray:
    """Boolean [Sq', Sk] array: True where query row i may attend to key j.

    Causal masking is aligned to the bottom-right corner: key j is visible to query i
    iff j <= i + (Sk - Sq).  For square problems this is the usual j <= i.  (The
    "FlashAttention_02" page leaves square vs non-square alignment to the
    implementation's documentation; this is the reading taken.)  ``q_index`` selects
    absolute query rows (default: all Sq rows).
    """
    qi = np.arange(Sq) if q_index is None else np.asarray(q_index, dtype=np.int64)
    if not causal:
        return np.ones((qi.shape[0], Sk), dtype=bool)
    kj = np.arange(Sk)
    return kj[None, :] <= (qi[:, None] + (Sk - Sq))


def scores(q, k, scale, causal=False, Sq_total=None, q_index=None):
    """Scaled, masked score matrix S [..., Sq', Sk] in float64 (masked entries -inf)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    Sq = q.shape[-2] if Sq_total is None else Sq_total
    s = np.float64(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    keep = visible_mask(Sq, k.shape[-2], causal, q_index)
    return np.where(keep, s, -np.inf)


def _row_softmax_parts(s):
    """(m, P, l) of a masked score matrix; fully masked rows give m=-inf, P=0, l=0."""
    m = np.max(s, axis=-1) if s.shape[-1] > 0 else np.full(s.shape[:-1], -np.inf)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    p = np.where(np.isfinite(s), np.exp(s - m_safe[..., None]), 0.0)
    l = np.sum(p, axis=-1)
    return m, p, l


def softmax_probs(q, k, scale, causal=False, Sq_total=None, q_index=None):
    """Attention probabilities P = softmax(S) [..., Sq', Sk]; fully masked rows are 0."""
    _, p, l = _row_softmax_parts(scores(q, k, scale, causal, Sq_total, q_index))
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(l[..., None] > 0, p / np.where(l > 0, l, 1.0)[..., None], 0.0)


def attention(q, k, v, scale, causal=False, Sq_total=None, q_index=None):
    """Exact attention: returns (O [..., Sq', d], lse [..., Sq']) in float64.

    ``Sq_total``/``q_index`` let a caller evaluate a sample of rows of a larger problem
    with the right causal alignment (rows ``q_index`` of a problem with ``Sq_total``
    query rows; ``q`` then holds just those rows).
    """
    v = np.asarray(v, dtype=np.float64)
    m, p, l = _row_softmax_parts(scores(q, k, scale, causal, Sq_total, q_index))
    pv = np.matmul(p, v)
    empty = ~(l > 0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(empty[..., None], 0.0, pv / np.where(empty, 1.0, l)[..., None])
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return o, lse


# ----------------------------------------------------------------------------- split-K
def split_bounds(Sk: int, n: int):
    """Key ranges of an n-way split: chunk size C = ceil(Sk/n), chunk s = [s*C, min(Sk,(s+1)*C)).

    Chunks past the end are empty (start == end == Sk).  For the page's four keys and
    n=2 this gives {0,1} and {2,3}, the two blocks of the worked example; n=3 leaves
    the third chunk empty (the empty tail block the page asks to cover).
    """
    if n < 1:
        raise ValueError("n must be >= 1")
    C = -(-Sk // n)
    out = []
    for s in range(n):
        a = min(Sk, s * C)
        b = min(Sk, (s + 1) * C)
        out.append((a, b))
    return out


def partial_state(q, k, v, scale, start, end, causal=False, Sq_total=None, q_index=None):
    """Local softmax state of keys [start, end): (m, l, u).

    m = max of the chunk's visible scaled scores (-inf if none), l = sum exp(S - m),
    u = sum exp(S - m) v (not divided by l).  An empty or fully masked chunk is
    (-inf, 0, 0).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Sq = q.shape[-2] if Sq_total is None else Sq_total
    Sk = k.shape[-2]
    s = scores(q, k, scale, causal, Sq, q_index)
    keep = np.zeros(Sk, dtype=bool)
    keep[start:end] = True
    s = np.where(keep, s, -np.inf)
    m, p, l = _row_softmax_parts(s)
    u = np.matmul(p, v)
    return m, l, u


def split_states(q, k, v, scale, n, causal=False, Sq_total=None, q_index=None):
    """Local states of every chunk of an n-way key split, as a list of (m, l, u)."""
    return [partial_state(q, k, v, scale, a, b, causal, Sq_total, q_index)
            for (a, b) in split_bounds(np.asarray(k).shape[-2], n)]


def merge_states(states):
    """Combine chunk states into (O, lse).

    M = max_s m_s; every chunk is rescaled by w_s = exp(m_s - M) (0 for an empty chunk);
    L = sum w_s l_s; O = sum w_s u_s / L; lse = M + ln L.  When every chunk is empty the
    row has no visible key: O = 0, lse = -inf.
    """
    ms = np.stack([s[0] for s in states])
    ls = np.stack([s[1] for s in states])
    us = np.stack([s[2] for s in states])
    M = np.max(ms, axis=0)
    finite = np.isfinite(M)
    M_safe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(ms), np.exp(ms - M_safe[None]), 0.0)
    L = np.sum(w * ls, axis=0)
    U = np.sum(w[..., None] * us, axis=0)
    empty = ~(L > 0)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(empty[..., None], 0.0, U / np.where(empty, 1.0, L)[..., None])
        lse = np.where(empty, -np.inf, M + np.log(np.where(empty, 1.0, L)))
    return o, lse


def naive_average(states):
    """The wrong combination the page warns about: normalise each chunk, then average.

    Kept only as a negative control (the page prints the value it gives for the worked
    example, which a correct merge must not reproduce).  Empty chunks are skipped.
    """
    outs = [u / l[..., None] for (m, l, u) in states if np.all(l > 0)]
    return sum(outs) / len(outs)


def attention_split(q, k, v, scale, n, causal=False, Sq_total=None, q_index=None):
    """Attention through an n-way key split and merge: (O, lse)."""
    return merge_states(split_states(q, k, v, scale, n, causal, Sq_total, q_index))


# ----------------------------------------------------------------------------- ragged batch
def attention_varlen(q, k, v, cu_q, cu_k, scale, causal=False):
    """Exact attention of a ragged batch: (O [H, total_q, d], lse [H, total_q]).

    Variable-length sequences packed as ragged tensors ("Inside FlashAttention-3" page,
    section 7.2): q is [H, total_q, d], k and v are [H, total_k, d]; sequence b owns
    query rows cu_q[b]:cu_q[b+1] and key rows cu_k[b]:cu_k[b+1] of every head and
    attends to its own keys only, with the causal mask aligned to its own bottom-right
    corner.  Each sequence is the plain definition above applied to its slices; a
    sequence with no keys gets O = 0, lse = -inf.  Rows that no sequence covers are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    H, Tq, d = q.shape
    o = np.full((H, Tq, d), np.nan)
    lse = np.full((H, Tq), np.nan)
    for b in range(len(cu_q) - 1):
        a, e = int(cu_q[b]), int(cu_q[b + 1])
        ka, ke = int(cu_k[b]), int(cu_k[b + 1])
        if e <= a:
            continue
        o[:, a:e], lse[:, a:e] = attention(q[:, a:e], k[:, ka:ke], v[:, ka:ke], scale, causal)
    return o, lse


def flops(B: int, H: int, Sq: int, Sk: int, d: int, causal: bool) -> float:
    """Counted FLOPs of one forward: 4*B*H*Sq*Sk*d, halved when causal."""
    f = 4.0 * B * H * Sq * Sk * d
    return f / 2.0 if causal else f


__all__.append("flops")
