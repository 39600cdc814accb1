"""Seeded synthetic inputs for exact attention, shared by the oracle side and the GPU side.

This module draws the random tensors and rounds them to the storage format that the
GPU consumes (fp32, bf16 bit patterns, or OCP FP8 E4M3 codes plus one fp32 scale per
tensor).  It holds none of the attention arithmetic: no scores, no softmax, no
reduction.  Both sides receive the very same bits; the oracle upcasts them exactly to
float64, the GPU library reads them as stored.

Recipe (no public dataset is named by the pages, so every workload is synthetic):
  * ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal(dtype=float32)``,
    drawn in the order Q, K, V, each of shape [B, H, S, d] (row-major).
  * Optional "hot rows": exactly ceil(frac * B*H*Sq) flat (b, h, row) indices of Q are
    chosen without replacement from the same generator (after V) and multiplied by
    ``hot_scale`` in fp32, *before* rounding.  This stresses the running-max shift that
    the online softmax must absorb (very large scores, "FlashAttention_02" page,
    section on correctness and deployment boundaries).
  * bf16: round-to-nearest-even from fp32.
  * fp8: per-tensor scale = amax / 448 (fp32), code = RNE(x / scale) in E4M3FN with
    saturation to +-448 (the FP8 format the "Inside FlashAttention-3" page names in its
    BF16/FP8 section; E4M3FN is the OCP flavour gfx950's FP8 MFMA consumes).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_round_bits", "bf16_bits_to_f32", "e4m3_decode", "e4m3_encode",
    "E4M3_MAX", "AttentionInputs", "make_attention_inputs", "worked_example_inputs",
    "WORKED_SCORES", "WORKED_VALUES",
]

E4M3_MAX = 448.0

# The one worked example printed on the "FlashAttention_02" page (split-K section):
# four scores and four scalar values for a single query row.
WORKED_SCORES = (1.0, 2.0, 4.0, 0.0)
WORKED_VALUES = (2.0, 5.0, 1.0, 9.0)


# ----------------------------------------------------------------------------- bf16
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN maps to a quiet NaN; +-inf and values that round past the largest finite bf16
    become +-inf, as IEEE rounding prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = r.copy()
        r[nan] = ((u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040))
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exactly equal fp32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- e4m3
def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (sign | 4-bit exponent, bias 7 | 3-bit mantissa).

    Exponent field 0 encodes subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN
    (the format has no infinities), every other code is normal (1 + m/8) * 2^(e-7).
    """
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3_VALUES = _e4m3_table()
_E4M3_POS = _E4M3_VALUES[:0x7F]  # codes 0..126: non-negative finite values, increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes (uint8) -> exactly equal fp32 values."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)].astype(np.float32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Real values -> E4M3FN codes: round to nearest, ties to the even code, saturate to +-448.

    NaN maps to the NaN code 0x7F (sign kept).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first value >= a
    hi = np.clip(hi, 0, len(_E4M3_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_E4M3_POS) - 1)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    nan = np.isnan(x)
    if nan.any():
        code[nan] = np.where(np.signbit(x[nan]), 0xFF, 0x7F)
    return code


# ----------------------------------------------------------------------------- inputs
@dataclass
class AttentionInputs:
    """One seeded attention problem in storage format plus its exact fp64 values.

    ``q``, ``k``, ``v`` are what the GPU library reads: float32 arrays (dtype 'f32'),
    uint16 bf16 bit patterns ('bf16') or uint8 E4M3 codes ('fp8'), all [B, H, S, d].
    ``q64``, ``k64``, ``v64`` are the real numbers those bits stand for, including the
    per-tensor fp8 scale, as float64.  ``scales`` holds (q, k, v) fp32 descales (1.0
    unless fp8).
    """
    dtype: str
    B: int
    H: int
    Sq: int
    Sk: int
    d: int
    seed: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q64: np.ndarray
    k64: np.ndarray
    v64: np.ndarray
    scales: tuple = (1.0, 1.0, 1.0)
    hot_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int64))


def _to_storage(x: np.ndarray, dtype: str):
    """Round fp32 ``x`` to the storage format; returns (stored, exact fp64 value, scale)."""
    if dtype == "f32":
        return x, x.astype(np.float64), 1.0
    if dtype == "bf16":
        bits = bf16_round_bits(x)
        return bits, bf16_bits_to_f32(bits).astype(np.float64), 1.0
    if dtype == "fp8":
        amax = float(np.max(np.abs(x))) if x.size else 0.0
        scale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
        codes = e4m3_encode(x.astype(np.float64) / np.float64(scale))
        val = e4m3_decode(codes).astype(np.float64) * np.float64(scale)
        return codes, val, float(scale)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_attention_inputs(B: int, H: int, Sq: int, Sk: int, d: int, seed: int,
                          dtype: str = "bf16", hot_row_frac: float = 0.0,
                          hot_scale: float = 30.0) -> AttentionInputs:
    """Draw Q [B,H,Sq,d], K and V [B,H,Sk,d] i.i.d. N(0,1) from ``seed`` and round them."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Sq, d), dtype=np.float32)
    k = rng.standard_normal((B, H, Sk, d), dtype=np.float32)
    v = rng.standard_normal((B, H, Sk, d), dtype=np.float32)
    hot = np.zeros(0, dtype=np.int64)
    if hot_row_frac > 0.0:
        nrows = B * H * Sq
        nhot = int(math.ceil(hot_row_frac * nrows))
        hot = np.sort(rng.choice(nrows, size=nhot, replace=False)).astype(np.int64)
        qf = q.reshape(nrows, d)
        qf[hot] = qf[hot] * np.float32(hot_scale)
    qs, q64, sq = _to_storage(q, dtype)
    ks, k64, sk = _to_storage(k, dtype)
    vs, v64, sv = _to_storage(v, dtype)
    return AttentionInputs(dtype, B, H, Sq, Sk, d, seed, qs, ks, vs, q64, k64, v64,
                           (sq, sk, sv), hot)


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """``n`` sequence lengths drawn uniformly from [lo, hi] (int64), seeded."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=n).astype(np.int64)


def cu_seqlens(lengths) -> np.ndarray:
    """Offsets [0, l0, l0+l1, ...] (int32) of sequences packed one after another."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def make_varlen_inputs(lens_q, lens_k, H: int, d: int, seed: int, dtype: str = "bf16"):
    """A ragged batch packed head-major: Q [H, sum(lens_q), d], K and V [H, sum(lens_k), d],
    drawn and rounded exactly like ``make_attention_inputs`` with B = 1 (one fp8 scale per
    packed tensor).  Returns (AttentionInputs with [1, H, total, d] arrays, cu_q, cu_k)."""
    cu_q, cu_k = cu_seqlens(lens_q), cu_seqlens(lens_k)
    inp = make_attention_inputs(1, H, max(int(cu_q[-1]), 1), max(int(cu_k[-1]), 1), d, seed, dtype)
    return inp, cu_q, cu_k


def worked_example_inputs(d: int = 64, dtype: str = "bf16") -> AttentionInputs:
    """The page's 1x4 worked example embedded in a d-dimensional head.

    One query q = e0, four keys k_j = s_j * e0 and values v_j = value_j * e0, with
    scale 1: the scaled scores are exactly (1, 2, 4, 0) and column 0 of the output is
    the softmax-weighted average of (2, 5, 1, 9); every other column is zero.  All of
    these numbers are exact in fp32, bf16 and E4M3, so no scale is needed for fp8.
    """
    q = np.zeros((1, 1, 1, d), dtype=np.float32)
    k = np.zeros((1, 1, 4, d), dtype=np.float32)
    v = np.zeros((1, 1, 4, d), dtype=np.float32)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, :, 0] = WORKED_SCORES
    v[0, 0, :, 0] = WORKED_VALUES
    if dtype == "f32":
        st = (q, k, v)
    elif dtype == "bf16":
        st = tuple(bf16_round_bits(t) for t in (q, k, v))
    elif dtype == "fp8":
        st = tuple(e4m3_encode(t) for t in (q, k, v))
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return AttentionInputs(dtype, 1, 1, 1, 4, d, -1, *st,
                           q.astype(np.float64), k.astype(np.float64),
                           v.astype(np.float64), (1.0, 1.0, 1.0))
