"""The seeded input generator: storage rounding against torch's CPU casts, determinism,
the hot-row recipe and the fp8 per-tensor scale.  No GPU."""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si


def _edge_f32():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    extra = np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875,  # bf16 ties
                      1e-40, -1e-42, 3.0e38, 3.4e38, np.inf, -np.inf,
                      65504.0, 1e-8, 2.0 ** -126, 2.0 ** -133], dtype=np.float32)
    return np.concatenate([x, extra, (x * 1e20).astype(np.float32), (x * 1e-20).astype(np.float32)])


def test_bf16_rounding_matches_torch_bit_for_bit():
    x = _edge_f32()
    ours = si.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = si.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_bf16_nan_stays_nan():
    bits = si.bf16_round_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(si.bf16_bits_to_f32(bits))[0]


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = si.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7F and 0xFF
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_rne_with_saturation():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 100.0,
        rng.standard_normal(5000) * 1e-3,
        [464.0, 480.0, 1000.0, -1e9, 0.0029296875, 2.0 ** -10, 2.0 ** -9 * 1.5, 0.0, -0.0,
         1.0625, 1.1875, 240.0, 248.0],  # ties
    ]).astype(np.float32)
    ours = si.e4m3_encode(x.astype(np.float64))
    clamped = torch.from_numpy(x).clamp(-si.E4M3_MAX, si.E4M3_MAX)
    ref = clamped.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # signed zero: torch keeps the sign of -0.0 and of values that round to zero
    np.testing.assert_array_equal(ours, ref)
    assert si.e4m3_encode(np.array([464.0]))[0] == 0x7E
    assert si.e4m3_decode(si.e4m3_encode(np.array([0.0029296875])))[0] == 0.00390625


def test_inputs_are_deterministic_per_seed():
    a = si.make_attention_inputs(1, 2, 16, 24, 8, seed=5, dtype="bf16")
    b = si.make_attention_inputs(1, 2, 16, 24, 8, seed=5, dtype="bf16")
    c = si.make_attention_inputs(1, 2, 16, 24, 8, seed=6, dtype="bf16")
    for t in ("q", "k", "v"):
        np.testing.assert_array_equal(getattr(a, t), getattr(b, t))
    assert not np.array_equal(a.q, c.q)
    assert a.q.shape == (1, 2, 16, 8) and a.k.shape == (1, 2, 24, 8)
    assert a.q.dtype == np.uint16


def test_f32_inputs_are_standard_normal_draws_in_order_q_k_v():
    a = si.make_attention_inputs(1, 1, 4, 5, 3, seed=11, dtype="f32")
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 1, 4, 3), dtype=np.float32)
    k = rng.standard_normal((1, 1, 5, 3), dtype=np.float32)
    v = rng.standard_normal((1, 1, 5, 3), dtype=np.float32)
    np.testing.assert_array_equal(a.q, q)
    np.testing.assert_array_equal(a.k, k)
    np.testing.assert_array_equal(a.v, v)
    np.testing.assert_array_equal(a.q64, q.astype(np.float64))


def test_hot_rows_recipe():
    B, H, Sq, d = 2, 3, 50, 8
    plain = si.make_attention_inputs(B, H, Sq, Sq, d, seed=3, dtype="f32")
    hot = si.make_attention_inputs(B, H, Sq, Sq, d, seed=3, dtype="f32", hot_row_frac=0.01)
    n = math.ceil(0.01 * B * H * Sq)
    assert hot.hot_rows.size == n == len(set(hot.hot_rows.tolist()))
    pq = plain.q.reshape(-1, d)
    hq = hot.q.reshape(-1, d)
    mask = np.zeros(B * H * Sq, dtype=bool)
    mask[hot.hot_rows] = True
    np.testing.assert_array_equal(hq[~mask], pq[~mask])
    np.testing.assert_array_equal(hq[mask], pq[mask] * np.float32(30.0))
    np.testing.assert_array_equal(hot.k, plain.k)


def test_fp8_scale_and_exact_values():
    a = si.make_attention_inputs(1, 2, 32, 64, 16, seed=4, dtype="fp8")
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 32, 16), dtype=np.float32)
    sq = np.float32(np.abs(q).max() / si.E4M3_MAX)
    assert a.scales[0] == float(sq)
    assert a.q.dtype == np.uint8
    np.testing.assert_array_equal(a.q64, si.e4m3_decode(a.q).astype(np.float64) * float(sq))
    # the element of largest magnitude lands on the largest code
    assert np.abs(si.e4m3_decode(a.q)).max() == si.E4M3_MAX
    # quantisation error is within half a step of the format (relative 2^-4) or the subnormal step
    err = np.abs(a.q64 - q.astype(np.float64))
    assert np.all(err <= np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10 * float(sq)) + 1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_worked_example_embedding_is_exact(dtype):
    a = si.worked_example_inputs(64, dtype)
    dec = {"f32": lambda t: t, "bf16": si.bf16_bits_to_f32, "fp8": si.e4m3_decode}[dtype]
    np.testing.assert_array_equal(dec(a.k)[0, 0, :, 0], si.WORKED_SCORES)
    np.testing.assert_array_equal(dec(a.v)[0, 0, :, 0], si.WORKED_VALUES)
    assert dec(a.q)[0, 0, 0, 0] == 1.0 and np.count_nonzero(dec(a.q)) == 1
