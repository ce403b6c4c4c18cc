"""GPU parity of moe_rank_to_expert_reorder against the oracle (bit-exact)."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import bits, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run(moe, x, counts, R, El, N=None, rows=True):
    if N is None:
        N = x.shape[0]
    print(f"reorder R={R} E_local={El} N={N} H={x.shape[1] if rows else 0}", flush=True)
    got = moe.reorder_alloc(to_dev_bf16(x) if rows else None, to_dev(counts), R, El, N, rows=rows)
    torch.cuda.synchronize()
    ref = oracle.reorder(x if rows else None, counts, R, El, N, rows=rows)
    for k in ("perm", "inv_perm", "tokens_per_expert", "expert_offsets"):
        np.testing.assert_array_equal(got[k].cpu().numpy(), ref[k], err_msg=k)
    if rows:
        total = int(counts.sum())
        np.testing.assert_array_equal(bits(got["y"][:total]), ref["y"][:total])


@pytest.mark.parametrize("R,El,N,H,seed", [
    (1, 1, 1, 8, 0), (1, 9, 500, 16, 1), (6, 1, 333, 24, 2), (8, 32, 4000, 136, 3),
    (3, 5, 0, 8, 4), (16, 64, 20000, 8, 5), (5, 205, 3000, 8, 7), (256, 256, 70000, 8, 6),
])
def test_reorder_random(moe_lib, R, El, N, H, seed):
    counts = W.make_rank_major_counts(R, El, N, seed)
    _run(moe_lib, W.make_tokens(N, H, seed), counts, R, El)


def test_reorder_capacity_and_empty_blocks(moe_lib):
    counts = np.array([0, 5, 0, 0, 3, 0, 0, 0, 7], np.int32)  # R = 3, E_local = 3
    x = W.make_tokens(20, 16, 1)
    _run(moe_lib, x, counts, 3, 3, N=20)          # 15 rows used, 5 rows of capacity
    _run(moe_lib, x[:15], np.zeros(9, np.int32), 3, 3, N=15)


def test_reorder_config4(moe_lib):
    g = W.gen_c4()
    c = g["cfg"]
    _run(moe_lib, g["x_rank_major"], g["counts"], c["R"], c["E_local"])
