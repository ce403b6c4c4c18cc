"""Pins of the oracle's grouped SwiGLU FFN: numpy fp64 matmul and scipy's
logistic function (library routines) for a dense FFN per expert, and closed
forms (zero gate, zero up projection, exact scaling)."""
import numpy as np
import pytest
from scipy.special import expit

import moe_workloads as W
import oracle


def _dense_ffn(x_bits, wg_bits, wu_bits, wd_bits):
    x = W.f32_from_bf16(x_bits).astype(np.float64)
    wg = W.f32_from_bf16(wg_bits).astype(np.float64)
    wu = W.f32_from_bf16(wu_bits).astype(np.float64)
    wd = W.f32_from_bf16(wd_bits).astype(np.float64)
    g = np.matmul(x, wg)
    u = np.matmul(x, wu)
    h = g * expit(g) * u
    return h, np.matmul(h, wd)


def test_single_expert_is_dense_ffn():
    rng = np.random.default_rng(0)
    N, H, I = 37, 48, 40
    x = W.normal_bf16(rng, (N, H))
    wg = W.normal_bf16(rng, (1, H, I), 0.1)
    wu = W.normal_bf16(rng, (1, H, I), 0.1)
    wd = W.normal_bf16(rng, (1, I, H), 0.1)
    h, y = oracle.grouped_swiglu(x, np.array([0, N], np.int32), wg, wu, wd)
    hr, yr = _dense_ffn(x, wg[0], wu[0], wd[0])
    np.testing.assert_allclose(h, hr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-12)


def test_groups_use_their_own_expert():
    rng = np.random.default_rng(1)
    E, H, I = 5, 32, 24
    counts = np.array([3, 0, 7, 1, 0], np.int32)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(off[-1]) + 2   # two capacity rows past the last group stay untouched
    x = W.normal_bf16(rng, (N, H))
    wg = W.normal_bf16(rng, (E, H, I), 0.1)
    wu = W.normal_bf16(rng, (E, H, I), 0.1)
    wd = W.normal_bf16(rng, (E, I, H), 0.1)
    h, y = oracle.grouped_swiglu(x, off, wg, wu, wd)
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b > a:
            hr, yr = _dense_ffn(x[a:b], wg[e], wu[e], wd[e])
            np.testing.assert_allclose(h[a:b], hr, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(y[a:b], yr, rtol=1e-12, atol=1e-12)
    assert np.all(y[off[-1]:] == 0) and np.all(h[off[-1]:] == 0)


def test_closed_forms():
    rng = np.random.default_rng(2)
    N, H, I = 9, 16, 8
    x = W.normal_bf16(rng, (N, H))
    wg = W.normal_bf16(rng, (1, H, I), 0.3)
    wu = W.normal_bf16(rng, (1, H, I), 0.3)
    wd = W.normal_bf16(rng, (1, I, H), 0.3)
    off = np.array([0, N], np.int32)
    zero = np.zeros_like(wg)
    h0, y0 = oracle.grouped_swiglu(x, off, zero, wu, wd)   # silu(0) = 0
    assert np.all(h0 == 0) and np.all(y0 == 0)
    h1, y1 = oracle.grouped_swiglu(x, off, wg, zero, wd)   # u = 0
    assert np.all(h1 == 0) and np.all(y1 == 0)
    h, y = oracle.grouped_swiglu(x, off, wg, wu, wd)
    two = W.bf16_from_f32(np.float32(2.0) * W.f32_from_bf16(wd))  # exact doubling in bf16
    _, y2 = oracle.grouped_swiglu(x, off, wg, wu, two)
    np.testing.assert_array_equal(y2, 2 * y)
    twou = W.bf16_from_f32(np.float32(2.0) * W.f32_from_bf16(wu))
    h3, _ = oracle.grouped_swiglu(x, off, wg, twou, wd)
    np.testing.assert_array_equal(h3, 2 * h)
    # silu(g) ~ g for large g: a huge positive gate makes h ~ g * u
    xg = W.bf16_from_f32(np.abs(W.f32_from_bf16(x)) + 1.0)
    ones = W.bf16_from_f32(np.full((1, H, I), 4.0, np.float32))
    hb, _ = oracle.grouped_swiglu(xg, off, ones, wu, wd)
    g = 4.0 * W.f32_from_bf16(xg).astype(np.float64).sum(1, keepdims=True)
    u = W.f32_from_bf16(xg).astype(np.float64) @ W.f32_from_bf16(wu[0]).astype(np.float64)
    np.testing.assert_allclose(hb, g * u, rtol=1e-12)


def test_swiglu_row_matches_grouped():
    rng = np.random.default_rng(3)
    H, I = 20, 12
    x = W.normal_bf16(rng, (4, H))
    wg = W.normal_bf16(rng, (2, H, I), 0.2)
    wu = W.normal_bf16(rng, (2, H, I), 0.2)
    wd = W.normal_bf16(rng, (2, I, H), 0.2)
    h, y = oracle.grouped_swiglu(x, np.array([0, 1, 4], np.int32), wg, wu, wd)
    hr, yr = oracle.swiglu_row(x[2], wg[1], wu[1], wd[1])
    np.testing.assert_array_equal(h[2], hr)
    np.testing.assert_array_equal(y[2], yr)


def test_rejects_bad_offsets():
    x = np.zeros((4, 8), np.uint16)
    w = np.zeros((2, 8, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.grouped_swiglu(x, np.array([0, 3, 2], np.int32), w, w, w)
    with pytest.raises(ValueError):
        oracle.grouped_swiglu(x, np.array([0, 3, 5], np.int32), w, w, w)
