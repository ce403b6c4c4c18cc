"""Pins of the oracle's unpermute-combine: the exact round trip of the
permute, torch's bf16 rounding of K*x (library routine), the closed forms of
the zero / copy / constant experts and of the unweighted shared term, the
column-split invariance of hidden-dim sharding, and the fused reorder map."""
import json
import os

import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_round_f32(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _z(bits):
    """Map -0 to +0: a sum that cancels exactly is +0, a product with 0 may be -0."""
    b = np.array(bits, dtype=np.uint16, copy=True)
    b[b == 0x8000] = 0
    return b


def _distinct_ids(rng, T, E, K):
    return np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)


@pytest.mark.parametrize("T,E,H", [(1, 1, 8), (100, 7, 40), (257, 16, 64)])
def test_top1_roundtrip_is_exact(T, E, H):
    rng = np.random.default_rng(T)
    x = W.normal_bf16(rng, (T, H))
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    p = oracle.permute(x, ids, E)
    out, _ = oracle.combine(p["permuted"], p["row_of_slot"], ids, np.ones((T, 1), np.float32), E)
    np.testing.assert_array_equal(out, x)


@pytest.mark.parametrize("K", [2, 3, 6, 8])
def test_topk_unit_probs_gives_rne_of_k_x(K):
    rng = np.random.default_rng(K)
    T, E, H = 64, 10, 32
    x = W.normal_bf16(rng, (T, H))
    ids = _distinct_ids(rng, T, E, K)
    p = oracle.permute(x, ids, E)
    out, _ = oracle.combine(p["permuted"], p["row_of_slot"], ids, np.ones((T, K), np.float32), E)
    # K * x is exact in fp32 for K <= 16, so torch's fp32 -> bf16 RNE is the reference
    np.testing.assert_array_equal(out, _torch_round_f32(np.float32(K) * W.f32_from_bf16(x)))


def test_normalised_probs_return_x_within_an_ulp():
    g = W.gen_c1(with_weights=False)
    x, ids, probs = g["x"], g["expert_ids"], g["probs"]
    p = oracle.permute(x, ids, g["cfg"]["E"])
    out, out64 = oracle.combine(p["permuted"], p["row_of_slot"], ids, probs, g["cfg"]["E"])
    xf = W.f32_from_bf16(x).astype(np.float64)
    np.testing.assert_allclose(out64, xf * probs.astype(np.float64).sum(1, keepdims=True),
                               rtol=1e-15, atol=1e-300)
    assert np.all(np.abs(W.f32_from_bf16(out) - xf) <= np.abs(xf) * 2**-7 + 1e-30)


def _special_setup(rng, T=32, K=4, H=24, E=6, Z=2, C=3, Nc=2):
    x = W.normal_bf16(rng, (T, H))
    eo = W.normal_bf16(rng, (T * K, H))
    ori = W.normal_bf16(rng, (T, H))
    shared = W.normal_bf16(rng, (T, H))
    cv = W.uniform_bf16(rng, (Nc, H), -1, 1)
    return x, eo, ori, shared, cv


def test_zero_experts_leave_shared_only():
    rng = np.random.default_rng(5)
    T, K, H, E, Z, C, Nc = 32, 4, 24, 6, 2, 3, 2
    _, eo, ori, shared, cv = _special_setup(rng)
    ids = rng.integers(E, E + Z, size=(T, K)).astype(np.int32)
    probs = rng.standard_normal((T, K)).astype(np.float32)
    ros = np.full((T, K), -1, np.int32)
    out, _ = oracle.combine(eo, ros, ids, probs, E, num_zero=Z, num_copy=C, num_const=Nc,
                            ori_x=ori, alpha1=np.ones(T, np.float32),
                            alpha2=np.ones(T, np.float32), alpha_strides=(1, 0, 0),
                            const_v=cv, shared_x=shared)
    np.testing.assert_array_equal(out, shared)    # added once, unweighted
    out0, _ = oracle.combine(eo, ros, ids, probs, E, num_zero=Z, num_copy=C, num_const=Nc,
                             ori_x=ori, alpha1=np.ones(T, np.float32),
                             alpha2=np.ones(T, np.float32), alpha_strides=(1, 0, 0), const_v=cv)
    assert np.all((out0 & 0x7FFF) == 0)


def test_copy_and_const_closed_forms():
    rng = np.random.default_rng(6)
    T, K, H, E, Z, C, Nc = 32, 4, 24, 6, 2, 3, 2
    _, eo, ori, shared, cv = _special_setup(rng)
    probs = (rng.integers(-8, 9, size=(T, K)) / 8.0).astype(np.float32)  # exact, signed
    ros = np.full((T, K), -1, np.int32)
    orif = W.f32_from_bf16(ori)
    psum = probs.sum(1, keepdims=True).astype(np.float32)
    # copy experts: sum_k p * ori_x, exact in fp32 here, so torch's RNE is the reference
    ids = rng.integers(E + Z, E + Z + C, size=(T, K)).astype(np.int32)
    out, _ = oracle.combine(eo, ros, ids, probs, E, num_zero=Z, num_copy=C, num_const=Nc,
                            ori_x=ori, alpha1=np.zeros(T, np.float32),
                            alpha2=np.zeros(T, np.float32), alpha_strides=(1, 0, 0), const_v=cv)
    np.testing.assert_array_equal(_z(out), _z(_torch_round_f32(psum * orif)))
    # const expert with alpha1 = 1, alpha2 = 0 behaves as copy
    idc = rng.integers(E + Z + C, E + Z + C + Nc, size=(T, K)).astype(np.int32)
    out1, _ = oracle.combine(eo, ros, idc, probs, E, num_zero=Z, num_copy=C, num_const=Nc,
                             ori_x=ori, alpha1=np.ones(T, np.float32),
                             alpha2=np.zeros(T, np.float32), alpha_strides=(1, 0, 0), const_v=cv)
    np.testing.assert_array_equal(_z(out1), _z(_torch_round_f32(psum * orif)))
    # alpha1 = 0, alpha2 = 1 and a single const id: p-sum times v[c]
    idc1 = np.full((T, K), E + Z + C + 1, np.int32)
    out2, _ = oracle.combine(eo, ros, idc1, probs, E, num_zero=Z, num_copy=C, num_const=Nc,
                             ori_x=ori, alpha1=np.zeros(T, np.float32),
                             alpha2=np.ones(T, np.float32), alpha_strides=(1, 0, 0), const_v=cv)
    np.testing.assert_array_equal(
        _z(out2), _z(_torch_round_f32(psum * W.f32_from_bf16(cv[1])[None, :])))
    # per-(c, h) coefficients in the page's (const_num, H) layout: strides (0, H, 1)
    a1 = rng.integers(-4, 5, size=(Nc, H)).astype(np.float32) / 4
    a2 = rng.integers(-4, 5, size=(Nc, H)).astype(np.float32) / 4
    idc0 = np.full((T, K), E + Z + C, np.int32)
    p1 = np.zeros((T, K), np.float32)
    p1[:, 0] = 1.0
    out3, out3_64 = oracle.combine(eo, ros, idc0, p1, E, num_zero=Z, num_copy=C, num_const=Nc,
                                   ori_x=ori, alpha1=a1, alpha2=a2, alpha_strides=(0, H, 1),
                                   const_v=cv)
    ref = a1[0][None, :].astype(np.float64) * orif + \
        a2[0][None, :].astype(np.float64) * W.f32_from_bf16(cv[0])[None, :]
    np.testing.assert_array_equal(out3_64, ref)


def test_column_split_invariance_and_signs():
    rng = np.random.default_rng(7)
    T, K, E, H = 40, 3, 9, 64
    x = W.normal_bf16(rng, (T, H))
    ids = _distinct_ids(rng, T, E, K)
    probs = rng.standard_normal((T, K)).astype(np.float32)
    shared = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    full, _ = oracle.combine(p["permuted"], p["row_of_slot"], ids, probs, E, shared_x=shared)
    a, _ = oracle.combine(p["permuted"][:, :24], p["row_of_slot"], ids, probs, E,
                          shared_x=shared[:, :24])
    b, _ = oracle.combine(p["permuted"][:, 24:], p["row_of_slot"], ids, probs, E,
                          shared_x=shared[:, 24:])
    np.testing.assert_array_equal(np.concatenate([a, b], 1), full)
    neg, _ = oracle.combine(p["permuted"], p["row_of_slot"], ids, -probs, E,
                            shared_x=(shared ^ 0x8000).astype(np.uint16))
    np.testing.assert_array_equal(neg, full ^ 0x8000)


def test_row_map_is_the_fused_inverse_reorder():
    rng = np.random.default_rng(8)
    R, El, N, H, T, K = 3, 4, 60, 16, 20, 3
    cnt = W.make_rank_major_counts(R, El, N, 9)
    xrm = W.normal_bf16(rng, (N, H))
    r = oracle.reorder(xrm, cnt, R, El)
    src = rng.permutation(N)[:T * K].reshape(T, K).astype(np.int32)
    ids = np.zeros((T, K), np.int32)
    probs = rng.random((T, K)).astype(np.float32)
    direct, _ = oracle.combine(xrm, src, ids, probs, El)
    mapped, _ = oracle.combine(r["y"], src, ids, probs, El, row_map=r["inv_perm"])
    np.testing.assert_array_equal(mapped, direct)


def test_dropped_slots_and_example_ids():
    g = json.load(open(os.path.join(GOLD, "combine_v2_example_ids.json")))
    ids = np.array(g["expert_ids"], dtype=np.int32)
    E, T, K, H = g["moe_expert_num"], 8, 8, 32
    rng = np.random.default_rng(10)
    x = W.normal_bf16(rng, (T, H))
    ori = W.normal_bf16(rng, (T, H))
    probs = (rng.integers(-8, 9, size=(T, K)) / 8.0).astype(np.float32)
    p = oracle.permute(x, ids, E)
    zeros = np.zeros_like(p["permuted"])
    one = np.ones(T, np.float32)
    cv = W.uniform_bf16(rng, (1, H), -1, 1)
    out, _ = oracle.combine(zeros, p["row_of_slot"], ids, probs, E, num_zero=1, num_copy=1,
                            num_const=1, ori_x=ori, alpha1=one, alpha2=one,
                            alpha_strides=(1, 0, 0), const_v=cv)
    # with all expert rows zero only the copy slots (id 33) remain: sum p * ori_x
    pc = np.where(ids == 33, probs, 0).sum(1, keepdims=True).astype(np.float32)
    np.testing.assert_array_equal(_z(out), _z(_torch_round_f32(pc * W.f32_from_bf16(ori))))
    # an id past every expert range, or a row outside the buffer, contributes nothing
    bad = ids.copy()
    bad[0, 0] = 99
    ros = p["row_of_slot"].copy()
    ros[1, 0] = 10**6
    o1, _ = oracle.combine(p["permuted"], ros, bad, probs, E, num_zero=1, num_copy=1, num_const=1,
                           ori_x=ori, alpha1=one, alpha2=one, alpha_strides=(1, 0, 0), const_v=cv)
    probs2 = probs.copy()
    probs2[0, 0] = 0
    probs2[1, 0] = 0
    o2, _ = oracle.combine(p["permuted"], p["row_of_slot"], ids, probs2, E, num_zero=1,
                           num_copy=1, num_const=1, ori_x=ori, alpha1=one, alpha2=one,
                           alpha_strides=(1, 0, 0), const_v=cv)
    np.testing.assert_array_equal(o1, o2)


def test_missing_operands_are_rejected():
    ids = np.full((2, 1), 5, np.int32)
    eo = np.zeros((2, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.combine(eo, np.zeros((2, 1), np.int32), ids, np.ones((2, 1), np.float32), 4,
                       num_copy=2)
    with pytest.raises(ValueError):
        oracle.combine(eo, np.zeros((2, 1), np.int32), ids, np.ones((2, 1), np.float32), 4,
                       num_const=2, ori_x=np.zeros((2, 8), np.uint16))
