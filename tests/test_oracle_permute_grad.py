"""Pins of the oracle's permute backward (the index_put that accumulates the
gradients of repeated indices, per the twinkle grouped-matmul PR): the
scatter-add form over the permute's row -> slot map, the adjoint identity of
the permute as a linear map, the top-1 round trip, K identical copies summing
to K times the row (rounded by torch), dropped slots, and agreement with the
combine at unit weights."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle


def _routing(rng, T, K, E, special_frac=0.0):
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    if special_frac > 0:
        mask = rng.random((T, K)) < special_frac
        ids[mask] = E + rng.integers(0, 3, size=int(mask.sum()))   # ids past the real experts
    return ids


@pytest.mark.parametrize("T,K,E,H,seed,special", [
    (17, 3, 6, 24, 0, 0.0),
    (40, 8, 12, 16, 1, 0.2),
    (9, 1, 4, 8, 2, 0.0),
    (33, 16, 20, 8, 3, 0.1),
])
def test_scatter_add_form(T, K, E, H, seed, special):
    """index_put with accumulation: every permuted row's gradient is added to
    the token it came from (walking rows, not tokens)."""
    rng = np.random.default_rng(seed)
    ids = _routing(rng, T, K, E, special)
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    N = int(p["expert_offsets"][-1])
    d = W.normal_bf16(rng, p["permuted"].shape)
    ref = np.zeros((T, H))
    src_tok = p["sorted_slot"][:N] // K
    np.add.at(ref, src_tok, W.f32_from_bf16(d[:N]).astype(np.float64))
    dx, dx64 = oracle.permute_grad(d, p["row_of_slot"])
    np.testing.assert_allclose(dx64, ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(dx, oracle.f64_to_bf16(ref))


def test_adjoint_identity():
    """<permute(x), d> = <x, permute_grad(d)> for the permute's linear map."""
    rng = np.random.default_rng(11)
    T, K, E, H = 31, 4, 9, 40
    ids = _routing(rng, T, K, E, 0.15)
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    N = int(p["expert_offsets"][-1])
    d = W.normal_bf16(rng, p["permuted"].shape)
    _, dx64 = oracle.permute_grad(d, p["row_of_slot"])
    lhs = np.sum(W.f32_from_bf16(p["permuted"][:N]).astype(np.float64)
                 * W.f32_from_bf16(d[:N]).astype(np.float64))
    rhs = np.sum(W.f32_from_bf16(x).astype(np.float64) * dx64)
    assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs))


def test_top1_round_trip_is_exact():
    rng = np.random.default_rng(5)
    T, E, H = 50, 7, 32
    ids = _routing(rng, T, 1, E)
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    dx, _ = oracle.permute_grad(p["permuted"], p["row_of_slot"])
    np.testing.assert_array_equal(dx, x)


@pytest.mark.parametrize("K", [2, 3, 8, 16])
def test_k_copies_sum_to_k_times_the_row(K):
    """All K slots routed: the permuted rows are K copies of x[t], so d_x = K x,
    whose bf16 rounding torch computes from the (exact) fp32 product."""
    rng = np.random.default_rng(20 + K)
    T, E, H = 12, 2 * K + 1, 48
    ids = _routing(rng, T, K, E)
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    dx, _ = oracle.permute_grad(p["permuted"], p["row_of_slot"])
    kx = torch.from_numpy(W.f32_from_bf16(x) * np.float32(K)).to(torch.bfloat16)
    np.testing.assert_array_equal(dx, kx.view(torch.int16).numpy().view(np.uint16))


def test_dropped_slots_contribute_nothing():
    rng = np.random.default_rng(7)
    T, K, E, H = 6, 3, 5, 16
    ids = _routing(rng, T, K, E)
    ids[2, :] = E + 1          # a token with no real expert
    ids[4, 1] = -1             # a dropped slot
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    d = W.normal_bf16(rng, p["permuted"].shape)
    dx, dx64 = oracle.permute_grad(d, p["row_of_slot"])
    assert np.all(dx64[2] == 0) and np.all(dx[2] == 0)
    r0, r2 = p["row_of_slot"][4, 0], p["row_of_slot"][4, 2]
    want = W.f32_from_bf16(d[r0]).astype(np.float64) + W.f32_from_bf16(d[r2]).astype(np.float64)
    np.testing.assert_array_equal(dx64[4], want)


def test_equals_the_combine_at_unit_weights():
    """The permute backward is the combine with every probability 1 and no
    special or shared terms (two independently pinned oracle functions)."""
    rng = np.random.default_rng(9)
    T, K, E, H = 25, 5, 11, 24
    ids = _routing(rng, T, K, E)
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    d = W.normal_bf16(rng, p["permuted"].shape)
    dx, dx64 = oracle.permute_grad(d, p["row_of_slot"])
    out, out64 = oracle.combine(d, p["row_of_slot"], ids, np.ones((T, K), np.float32), E)
    np.testing.assert_allclose(dx64, out64, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(dx, out)
