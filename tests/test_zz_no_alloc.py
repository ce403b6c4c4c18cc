"""moe_permute_noalloc (count table in the library's own per-GPU array) against
moe_permute with a caller workspace, through the C ABI: every output
bit-exact, on two calls in a row, the second with a smaller input (and a
different count-table shape), then a third with a slot mask."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import bits, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

KEYS = ("permuted", "sorted_slot", "row_of_slot", "expert_counts", "expert_offsets")


def _outputs(T, K, E, H, dev):
    S = T * K
    return dict(permuted=torch.full((S, H), -1.0, dtype=torch.bfloat16, device=dev),
                sorted_slot=torch.full((S,), -7, dtype=torch.int32, device=dev),
                row_of_slot=torch.full((T, K), -7, dtype=torch.int32, device=dev),
                expert_counts=torch.full((E,), -7, dtype=torch.int32, device=dev),
                expert_offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=dev))


def _case(moe, T, K, E, H, seed, mask=None):
    print(f"permute_noalloc T={T} K={K} E={E} H={H} mask={mask is not None}", flush=True)
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    x = W.normal_bf16(rng, (T, H))
    dev = torch.device("cuda:0")
    xd, idd = to_dev_bf16(x), to_dev(ids)
    md = to_dev(mask) if mask is not None else None
    a = _outputs(T, K, E, H, dev)
    moe.moe_permute_noalloc(xd, idd, T, H, K, E, a["permuted"], a["sorted_slot"], a["row_of_slot"],
                            a["expert_counts"], a["expert_offsets"], active_mask=md)
    b = _outputs(T, K, E, H, dev)
    ws = moe.workspace(moe.moe_permute_workspace_size(T, K, E), dev)
    moe.moe_permute(xd, idd, T, H, K, E, b["permuted"], b["sorted_slot"], b["row_of_slot"],
                    b["expert_counts"], b["expert_offsets"], ws, active_mask=md)
    torch.cuda.synchronize()
    n = int(b["expert_offsets"][-1].item())
    for k in KEYS:
        ga = bits(a[k][:n]) if k == "permuted" else a[k].cpu().numpy()
        gb = bits(b[k][:n]) if k == "permuted" else b[k].cpu().numpy()
        np.testing.assert_array_equal(ga, gb, err_msg=k)
    ref = oracle.permute(x, ids, E, active_mask=mask)
    np.testing.assert_array_equal(a["row_of_slot"].cpu().numpy(), ref["row_of_slot"])
    np.testing.assert_array_equal(bits(a["permuted"][:n]), ref["permuted"][:n])


def test_permute_noalloc_matches_workspace_call(moe_lib):
    # the T=4096, E=64, K=6 workload's shape, then a smaller input with a
    # different count table, then a slot mask
    _case(moe_lib, 4096, 6, 64, 2048, 51)
    _case(moe_lib, 300, 2, 8, 128, 52)
    m = np.random.default_rng(53).random((1000, 4)) < 0.8
    _case(moe_lib, 1000, 4, 256, 64, 54, mask=m)
