"""GPU parity of moe_permute against the oracle: bit-exact indices, counts,
offsets and permuted rows."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import bits, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run_and_compare(moe, x, ids, E, rows=True):
    T, K = ids.shape
    print(f"permute T={T} K={K} E={E} H={x.shape[1] if rows else 0}", flush=True)
    xd = to_dev_bf16(x) if rows else None
    got = moe.permute_alloc(xd, to_dev(ids), E, rows=rows)
    torch.cuda.synchronize()
    ref = oracle.permute(x if rows else None, ids, E, rows=rows)
    np.testing.assert_array_equal(got["expert_counts"].cpu().numpy(), ref["expert_counts"])
    np.testing.assert_array_equal(got["expert_offsets"].cpu().numpy(), ref["expert_offsets"])
    np.testing.assert_array_equal(got["sorted_slot"].cpu().numpy(), ref["sorted_slot"])
    np.testing.assert_array_equal(got["row_of_slot"].cpu().numpy(), ref["row_of_slot"])
    if rows:
        n = int(ref["expert_offsets"][-1])
        np.testing.assert_array_equal(bits(got["permuted"][:n]), ref["permuted"][:n])
    return got, ref


@pytest.mark.parametrize("T,K,E,H,special,seed", [
    (1, 1, 1, 8, 0, 0),
    (5, 2, 3, 16, 0, 1),
    (300, 2, 8, 128, 0, 2),       # ragged: one chunk, partly filled
    (1100, 6, 64, 264, 0, 3),     # several chunks, H not a multiple of 64
    (3000, 8, 256, 64, 5, 4),     # special ids >= E mixed in
    (777, 16, 40, 32, 3, 5),      # K = 16
    (2049, 1, 1024, 8, 0, 6),     # E = 1024
    (8192, 4, 1024, 8, 0, 8),     # E = 1024 with a full count table (scan LDS past 64 KB)
    (4097, 4, 17, 8, 2, 7),
])
def test_permute_random(moe_lib, T, K, E, H, special, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E + special, size=(T, K)).astype(np.int32)
    if special:
        ids[::7, 0] = -1
    x = W.normal_bf16(rng, (T, H))
    _run_and_compare(moe_lib, x, ids, E)


def test_permute_skewed_and_empty_experts(moe_lib):
    ids, _ = W.make_routing(5000, 96, 6, seed=11, zipf_s=1.5, empty_experts=20)
    x = W.make_tokens(5000, 72, seed=12)
    got, ref = _run_and_compare(moe_lib, x, ids, 96)
    assert (ref["expert_counts"] == 0).sum() >= 20


def test_permute_degenerate(moe_lib):
    # all slots special
    ids = np.full((100, 3), 9, np.int32)
    _run_and_compare(moe_lib, W.make_tokens(100, 16, 1), ids, 4)
    # a single expert takes everything
    ids = np.zeros((513, 2), np.int32)
    _run_and_compare(moe_lib, W.make_tokens(513, 16, 2), ids, 7)
    # T = 0
    got = moe_lib.permute_alloc(torch.empty((0, 16), dtype=torch.bfloat16, device="cuda"),
                                torch.empty((0, 2), dtype=torch.int32, device="cuda"), 5)
    torch.cuda.synchronize()
    assert got["expert_offsets"].cpu().tolist() == [0] * 6
    assert got["expert_counts"].cpu().tolist() == [0] * 5


def test_permute_many_chunks(moe_lib):
    # more than 1024 * 256 * 8 slots: more slots per lane than the minimum
    T, K, E = 300000, 8, 128
    ids, _ = W.make_routing(T, E, K, seed=13)
    _run_and_compare(moe_lib, np.zeros((T, 8), np.uint16), ids, E, rows=False)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_permute_configs(moe_lib, cfg):
    kw = {1: dict(with_weights=False), 2: {}, 3: dict(with_weights=False)}[cfg]
    g = W.generate(cfg, **kw)
    _run_and_compare(moe_lib, g["x"], g["expert_ids"], g["cfg"]["E"])


def test_permute_config5_routing(moe_lib):
    g = W.gen_c5(with_rows=False)
    got, ref = _run_and_compare(moe_lib, np.zeros((g["cfg"]["T"], 8), np.uint16),
                                g["expert_ids"], g["cfg"]["E"], rows=False)
    assert int((ref["expert_counts"] == 0).sum()) == g["cfg"]["empty_experts"]


@pytest.mark.parametrize("T,K,E,H,special,seed", [
    (300, 2, 8, 128, 0, 21), (1100, 6, 64, 2056, 3, 22), (40, 16, 40, 32, 0, 23),
])
def test_permute_rows_applies_a_routing(moe_lib, T, K, E, H, special, seed):
    """moe_permute_rows moves a second tensor with the oracle's routing: its
    rows equal the oracle permute of that tensor; rows no slot names keep
    their contents."""
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E + special)), axis=1)[:, :K].astype(np.int32)
    x2 = W.normal_bf16(rng, (T, H))
    ref = oracle.permute(x2, ids, E)
    N = T * K
    n = int(ref["expert_offsets"][-1])
    print(f"permute_rows T={T} K={K} E={E} H={H} rows={n}", flush=True)
    out = torch.full((N, H), 3.0, dtype=torch.bfloat16, device="cuda")
    moe_lib.moe_permute_rows(to_dev_bf16(x2), to_dev(ref["row_of_slot"]), T, H, K, N, out)
    torch.cuda.synchronize()
    got = bits(out)
    np.testing.assert_array_equal(got[:n], ref["permuted"][:n])
    assert (got[n:] == W.bf16_from_f32(np.float32([3.0]))[0]).all()
