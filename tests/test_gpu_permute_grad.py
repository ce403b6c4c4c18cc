"""GPU parity of moe_permute_grad (the permute backward: each token's gradient is
the sum of its routed rows' gradients) against the oracle: the 1e-2 relative
bound in general, exact where the sum is exact in fp32."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_rel, bits, to_dev, to_dev_bf16, ulp_diff

pytestmark = pytest.mark.gpu


def _routing(rng, T, K, E, special_frac=0.0):
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    if special_frac > 0:
        mask = rng.random((T, K)) < special_frac
        ids[mask] = E + rng.integers(0, 3, size=int(mask.sum()))
    return ids


def _run(moe, d, ros):
    T, K = ros.shape
    print(f"permute_grad T={T} K={K} N={d.shape[0]} H={d.shape[1]}", flush=True)
    got = moe.permute_grad_alloc(to_dev_bf16(d), to_dev(ros))
    torch.cuda.synchronize()
    ref, ref64 = oracle.permute_grad(d, ros)
    got = bits(got)
    assert_rel(W.f32_from_bf16(got), ref64, 1e-2, "d_x")
    assert ulp_diff(got, ref) <= 1, "d_x: more than one bf16 ulp from the correctly rounded sum"
    return got, ref


@pytest.mark.parametrize("T,K,E,H,seed,special", [
    (1, 1, 1, 8, 0, 0.0), (300, 2, 8, 128, 1, 0.0), (1000, 6, 64, 264, 2, 0.1),
    (513, 8, 32, 4096, 3, 0.05), (64, 16, 20, 8200, 4, 0.0),
])
def test_permute_grad_random(moe_lib, T, K, E, H, seed, special):
    rng = np.random.default_rng(seed)
    ids = _routing(rng, T, K, E, special)
    p = oracle.permute(None, ids, E, rows=False)
    N = int(p["expert_offsets"][-1])
    _run(moe_lib, W.normal_bf16(rng, (max(N, 1), H)), p["row_of_slot"])


def test_permute_grad_round_trip_of_the_device_permute(moe_lib):
    """Top-1 on the device path: permute then its backward gives x back bit for bit."""
    rng = np.random.default_rng(8)
    T, E, H = 777, 13, 520
    x = W.normal_bf16(rng, (T, H))
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    p = moe_lib.permute_alloc(to_dev_bf16(x), to_dev(ids), E)
    dx = moe_lib.permute_grad_alloc(p["permuted"], p["row_of_slot"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(dx), x)


@pytest.mark.parametrize("K", [2, 8, 16])
def test_permute_grad_k_copies_exact(moe_lib, K):
    """Every slot routed and every row a copy of x[t]: d_x = K x, exact in fp32."""
    rng = np.random.default_rng(30 + K)
    T, E, H = 400, 2 * K + 3, 136
    ids = _routing(rng, T, K, E)
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    got, ref = _run(moe_lib, p["permuted"], p["row_of_slot"])
    np.testing.assert_array_equal(got, ref)


def test_permute_grad_dropped_and_empty(moe_lib):
    rng = np.random.default_rng(6)
    T, K, E, H = 200, 4, 10, 64
    ids = rng.integers(0, E + 3, size=(T, K)).astype(np.int32)
    ids[:7] = -1                      # tokens with nothing routed get zero rows
    p = oracle.permute(None, ids, E, rows=False)
    N = int(p["expert_offsets"][-1])
    got, _ = _run(moe_lib, W.normal_bf16(rng, (N, H)), p["row_of_slot"])
    assert np.all(got[:7] == 0)
    # nothing routed at all, and no tokens
    ros = np.full((5, 3), -1, np.int32)
    got, _ = _run(moe_lib, np.zeros((0, 16), np.uint16), ros)
    assert np.all(got == 0)
    out = moe_lib.permute_grad_alloc(torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda"),
                                     torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, 16)


def test_permute_grad_layer_size(moe_lib):
    """At the layer's size (T=8192, H=2048, top-8 of 256 experts, skewed routing)."""
    g = W.gen_c3(with_weights=False, with_x=False)
    c = g["cfg"]
    p = oracle.permute(None, g["expert_ids"], c["E"], rows=False)
    N = int(p["expert_offsets"][-1])
    rng = np.random.default_rng(12)
    _run(moe_lib, W.normal_bf16(rng, (N, c["H"])), p["row_of_slot"])
