"""Pins of the oracle's unpermute backward: central finite differences of the
oracle combine (d_probs), the adjoint identity of a linear map, the hidden-dim
sharding rules (Shard(1) for d_permuted, Partial() sum for d_probs), and exact
fp64 products for d_permuted."""
import numpy as np
import pytest

import moe_workloads as W
import oracle


def _setup(seed, T=24, K=3, E=7, H=40):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    # probs on a 2^-10 grid so that p +- 1 is exact in fp32
    probs = (rng.integers(-1024, 1025, size=(T, K)) / 1024.0).astype(np.float32)
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    perm = W.normal_bf16(rng, p["permuted"].shape)     # arbitrary expert outputs
    g = W.normal_bf16(rng, (T, H))
    return ids, probs, p, perm, g, E


def test_d_probs_is_the_finite_difference_of_the_combine():
    ids, probs, p, perm, g, E = _setup(0)
    gf = W.f32_from_bf16(g).astype(np.float64)
    _, dprobs, _, dprobs64 = oracle.unpermute_grad(g, perm, p["row_of_slot"], probs)
    T, K = probs.shape
    for t in range(0, T, 5):
        for k in range(K):
            pp, pm = probs.copy(), probs.copy()
            pp[t, k] += 1.0
            pm[t, k] -= 1.0
            _, op = oracle.combine(perm, p["row_of_slot"], ids, pp, E)
            _, om = oracle.combine(perm, p["row_of_slot"], ids, pm, E)
            fd = (np.sum(op * gf) - np.sum(om * gf)) / 2.0
            assert abs(fd - dprobs64[t, k]) <= 1e-10 * (1 + abs(fd))
    np.testing.assert_array_equal(dprobs, dprobs64.astype(np.float32))


def test_adjoint_identity():
    ids, probs, p, perm, g, E = _setup(1)
    _, out64 = oracle.combine(perm, p["row_of_slot"], ids, probs, E)
    _, dprobs, dperm64, dprobs64 = oracle.unpermute_grad(g, perm, p["row_of_slot"], probs)
    lhs = np.sum(out64 * W.f32_from_bf16(g))
    rhs = np.sum(W.f32_from_bf16(perm).astype(np.float64) * dperm64)
    rhs2 = np.sum(probs.astype(np.float64) * dprobs64)
    assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs))
    assert abs(lhs - rhs2) <= 1e-10 * (1 + abs(lhs))


def test_d_permuted_is_a_scaled_gather():
    ids, probs, p, perm, g, E = _setup(2)
    dperm, _, dperm64, _ = oracle.unpermute_grad(g, perm, p["row_of_slot"], probs)
    ros = p["row_of_slot"]
    T, K = probs.shape
    gf = W.f32_from_bf16(g).astype(np.float64)
    for t in range(T):
        for k in range(K):
            r = ros[t, k]
            np.testing.assert_array_equal(dperm64[r], probs[t, k].astype(np.float64) * gf[t])
    np.testing.assert_array_equal(dperm, oracle.f64_to_bf16(dperm64))


def test_hidden_dim_sharding_rules():
    ids, probs, p, perm, g, E = _setup(3, H=64)
    ros = p["row_of_slot"]
    dperm, _, _, dp64 = oracle.unpermute_grad(g, perm, ros, probs)
    a = oracle.unpermute_grad(g[:, :24], perm[:, :24], ros, probs)
    b = oracle.unpermute_grad(g[:, 24:], perm[:, 24:], ros, probs)
    np.testing.assert_array_equal(np.concatenate([a[0], b[0]], 1), dperm)   # Shard(1)
    np.testing.assert_allclose(a[3] + b[3], dp64, rtol=1e-12, atol=1e-12)   # Partial()


def test_special_slots_get_zero_and_untouched_rows_stay():
    ids, probs, p, perm, g, E = _setup(4)
    ros = p["row_of_slot"].copy()
    ros[0, 0] = -1
    init = np.full(perm.shape, 0x1234, np.uint16)
    dperm, dprobs, _, _ = oracle.unpermute_grad(g, perm, ros, probs, d_permuted_init=init)
    assert dprobs[0, 0] == 0.0
    freed = p["row_of_slot"][0, 0]
    assert np.all(dperm[freed] == 0x1234)
