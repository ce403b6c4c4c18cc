"""Pins of the oracle's grouped SwiGLU backward against the (independently
pinned) forward oracle: the loss L = <y, dy> is linear in W_down, W_up and in
h, so <dWd, Wd> = <dWu, Wu> = <dh, h> = L exactly; W_down and W_up elements
have exact central differences; x and W_gate elements (through the SiLU) are
checked against Richardson-extrapolated central differences on inputs whose
perturbations are exact in bf16; experts without rows get zero gradients."""
import numpy as np
import pytest

import moe_workloads as W
import oracle


def _grid_bf16(rng, shape, step, kmax):
    """Values k * step with |k| <= kmax: exact in bf16 for kmax < 2^8."""
    return W.bf16_from_f32((rng.integers(-kmax, kmax + 1, size=shape) * step).astype(np.float32))


def _setup(seed, counts=(5, 0, 7, 3), H=16, I=8):
    rng = np.random.default_rng(seed)
    E = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(off[-1]) + 2                                   # two rows past the last expert
    x = _grid_bf16(rng, (N, H), 2.0 ** -9, 200)            # |x| < 0.4
    wg = _grid_bf16(rng, (E, H, I), 2.0 ** -6, 100)        # |w| < 1.6
    wu = _grid_bf16(rng, (E, H, I), 2.0 ** -6, 100)
    wd = _grid_bf16(rng, (E, I, H), 2.0 ** -6, 100)
    dy = W.normal_bf16(rng, (N, H))
    return x, off, wg, wu, wd, dy


def _loss(x, off, wg, wu, wd, dy):
    _, y = oracle.grouped_swiglu(x, off, wg, wu, wd, want_h=False)
    return float(np.sum(y * W.f32_from_bf16(dy).astype(np.float64)))


def _set(a, idx, val):
    b = a.copy()
    b[idx] = W.bf16_from_f32(np.array([val], np.float32))[0]
    return b


def _cd(fn, a, idx, d):
    v = float(W.f32_from_bf16(np.array([a[idx]]))[0])
    return (fn(_set(a, idx, v + d)) - fn(_set(a, idx, v - d))) / (2 * d)


def test_linear_inputs_adjoint_identities():
    x, off, wg, wu, wd, dy = _setup(0)
    r = oracle.grouped_swiglu_grad(x, off, wg, wu, wd, dy)
    L = _loss(x, off, wg, wu, wd, dy)
    f = lambda b: W.f32_from_bf16(b).astype(np.float64)
    h, _ = oracle.grouped_swiglu(x, off, wg, wu, wd)
    for name, val in (("dwd", np.sum(r["dwd"] * f(wd))), ("dwu", np.sum(r["dwu"] * f(wu))),
                      ("dh", np.sum(r["dh"] * h))):
        assert abs(val - L) <= 1e-10 * (1 + abs(L)), name


def test_exact_central_differences_for_w_down_and_w_up():
    x, off, wg, wu, wd, dy = _setup(1)
    r = oracle.grouped_swiglu_grad(x, off, wg, wu, wd, dy)
    rng = np.random.default_rng(2)
    for _ in range(12):
        e, i, j = int(rng.choice([0, 2, 3])), int(rng.integers(8)), int(rng.integers(16))
        fd = _cd(lambda b: _loss(x, off, wg, wu, b, dy), wd, (e, i, j), 2.0 ** -6)
        assert abs(fd - r["dwd"][e, i, j]) <= 1e-9 * (1 + abs(fd))
        fd = _cd(lambda b: _loss(x, off, wg, b, wd, dy), wu, (e, j, i), 2.0 ** -6)
        assert abs(fd - r["dwu"][e, j, i]) <= 1e-9 * (1 + abs(fd))


def _richardson(fn, a, idx, d):
    return (4 * _cd(fn, a, idx, d / 2) - _cd(fn, a, idx, d)) / 3


def test_x_and_w_gate_against_extrapolated_differences():
    x, off, wg, wu, wd, dy = _setup(3)
    r = oracle.grouped_swiglu_grad(x, off, wg, wu, wd, dy)
    rng = np.random.default_rng(4)
    scale = np.sqrt(np.mean(r["dx"] ** 2)) + np.sqrt(np.mean(r["dwg"] ** 2))
    for _ in range(12):
        row, k = int(rng.integers(15)), int(rng.integers(16))
        fd = _richardson(lambda b: _loss(b, off, wg, wu, wd, dy), x, (row, k), 2.0 ** -6)
        assert abs(fd - r["dx"][row, k]) <= 1e-5 * (abs(fd) + scale), (row, k)
        e, i = int(rng.choice([0, 2, 3])), int(rng.integers(8))
        fd = _richardson(lambda b: _loss(x, off, b, wu, wd, dy), wg, (e, k, i), 2.0 ** -4)
        assert abs(fd - r["dwg"][e, k, i]) <= 1e-5 * (abs(fd) + scale), (e, k, i)


def test_empty_experts_and_rows_past_the_end():
    x, off, wg, wu, wd, dy = _setup(5)
    r = oracle.grouped_swiglu_grad(x, off, wg, wu, wd, dy)
    assert not r["dwg"][1].any() and not r["dwu"][1].any() and not r["dwd"][1].any()
    assert not r["dx"][int(off[-1]):].any()
    # a zero upstream gradient gives zero gradients everywhere
    z = oracle.grouped_swiglu_grad(x, off, wg, wu, wd, np.zeros_like(dy))
    assert not any(v.any() for v in z.values())
