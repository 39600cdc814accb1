"""Shared helpers of the GPU parity tests: device upload of seeded inputs, oracle
evaluation on all or on sampled rows, and the tolerance check.

Tolerances (from the stated parity bar): bf16 inputs max|dO| <= 1e-2 and mean|dO| <= 1e-3;
fp32 inputs max|dO| <= 1e-5; fp8 inputs max|dO| <= 5e-2; lse within 1e-3 on finite
entries, and -inf entries (rows with no visible key) must match exactly.  The bar states
no mean for fp8; the one used here, 1e-2, is the max bar over 5: the E4M3 rounding of the
probabilities (unit roundoff 2^-4) averages out over a row's keys, and the worst mean
measured (ragged batches with a handful of keys per row) is about 3e-3.
"""
import numpy as np
import torch

import oracle

TOL = {
    "f32": dict(max_o=1e-5, mean_o=1e-5, lse=1e-3),
    "bf16": dict(max_o=1e-2, mean_o=1e-3, lse=1e-3),
    "fp8": dict(max_o=5e-2, mean_o=1e-2, lse=1e-3),
}


def to_device(arr: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)
    raise ValueError(dtype)


def upload(inp, dev="cuda"):
    return tuple(to_device(t, inp.dtype, dev) for t in (inp.q, inp.k, inp.v))


def sample_rows(Sq: int, n: int, seed: int, must=()):
    """Sorted row indices: the given ones, tile edges, both ends, and random rows."""
    rng = np.random.default_rng(seed)
    base = {0, Sq - 1, min(Sq - 1, 127), min(Sq - 1, 128), Sq // 2, max(0, Sq - 129)}
    base |= {int(r) for r in must if 0 <= r < Sq}
    extra = rng.choice(Sq, size=min(Sq, n), replace=False)
    return np.array(sorted(base | {int(x) for x in extra}), dtype=np.int64)


def oracle_rows(inp, scale, causal, rows=None, heads=None):
    """Oracle (O, lse) for all heads (or the listed flat b*H+h heads) on all or sampled rows.

    Returns arrays shaped [nheads, nrows, d] and [nheads, nrows]."""
    B, H, Sq = inp.B, inp.H, inp.Sq
    q = inp.q64.reshape(B * H, Sq, inp.d)
    k = inp.k64.reshape(B * H, inp.Sk, inp.d)
    v = inp.v64.reshape(B * H, inp.Sk, inp.d)
    hs = range(B * H) if heads is None else heads
    outs, lses = [], []
    for h in hs:
        qq = q[h] if rows is None else q[h][rows]
        o, l = oracle.attention(qq, k[h], v[h], scale, causal, Sq_total=Sq, q_index=rows)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def check(name, o_gpu, lse_gpu, o_ref, lse_ref, dtype, tol=None):
    """Compare GPU results (numpy, fp32) against the oracle (fp64); returns the error stats."""
    t = dict(TOL[dtype]) if tol is None else tol
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{name}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    ref_inf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), ref_inf), f"{name}: -inf lse pattern differs"
    assert not np.any(np.isnan(lse_gpu)), f"{name}: NaN lse"
    lerr = np.abs(lse_gpu[~ref_inf] - lse_ref[~ref_inf])
    stats = dict(max_o=float(err.max()) if err.size else 0.0,
                 mean_o=float(err.mean()) if err.size else 0.0,
                 lse=float(lerr.max()) if lerr.size else 0.0)
    print(f"[{name}] max|dO|={stats['max_o']:.3e} mean|dO|={stats['mean_o']:.3e} "
          f"max|dlse|={stats['lse']:.3e}", flush=True)
    assert stats["max_o"] <= t["max_o"], f"{name}: max|dO| {stats['max_o']} > {t['max_o']}"
    assert stats["mean_o"] <= t["mean_o"], f"{name}: mean|dO| {stats['mean_o']} > {t['mean_o']}"
    assert stats["lse"] <= t["lse"], f"{name}: max|dlse| {stats['lse']} > {t['lse']}"
    return stats


def scale_for(d: int) -> float:
    """1/sqrt(d) rounded to fp32: the value both sides use."""
    return float(np.float32(1.0 / np.sqrt(d)))
