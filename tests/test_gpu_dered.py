"""GPU parity of the deredundency calls against the oracle: dispatch indices,
counts and total bit-exact; the whiteboard bit-exact where a row has at most
one source (a correctly rounded product per row on both sides, zero rows
elsewhere), and where several sources land on one row (the page's scatter-add
accumulates them) within the 1e-2 relative bound of the fp64 sum, and the same
bits on every run."""
import json
import os

import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_rel, bits, f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden", "dered_tiny.json")


def _indices(moe, c, start, iep, El, capacity):
    oep, E = c.shape
    print(f"dered indices oep={oep} E={E} start={start} iep={iep} El={El} cap={capacity}",
          flush=True)
    got = moe.dered_indices_alloc(to_dev(c), start, iep, El, capacity=capacity)
    torch.cuda.synchronize()
    idx, cbd, tot = oracle.dered_indices(c, start, iep, El, capacity=capacity)
    np.testing.assert_array_equal(got["indices"].cpu().numpy(), idx)
    np.testing.assert_array_equal(got["counts_by_dest"].cpu().numpy(), cbd)
    assert int(got["total"].item()) == tot
    return got, idx, tot


def test_dered_indices_fixtures(moe_lib):
    for case in json.load(open(GOLD))["cases"]:
        c = np.array(case["counts"], np.int32)
        _, idx, tot = _indices(moe_lib, c, case["expert_start"], case["iep_size"],
                               case["num_local"], int(c.sum()) + 3)
        np.testing.assert_array_equal(idx[:tot], case["indices"])


@pytest.mark.parametrize("oep,E,iep,El,start,seed", [
    (1, 8, 2, 4, 0, 0), (4, 64, 4, 8, 16, 1), (8, 256, 8, 4, 128, 2), (3, 10, 1, 1, 9, 3),
    (16, 1024, 8, 64, 0, 4), (64, 512, 2, 16, 480, 5),
])
def test_dered_indices_random(moe_lib, oep, E, iep, El, start, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 50, size=(oep, E)).astype(np.int32)
    c[rng.random((oep, E)) < 0.3] = 0
    c[0, start] = -4                                       # negative counts read as 0
    sel = int(np.maximum(c, 0)[:, start:start + iep * El].sum())
    _indices(moe_lib, c, start, iep, El, sel + 17)         # capacity past the total
    _indices(moe_lib, c, start, iep, El, max(sel // 2, 1))  # capacity below the total


def test_dered_empty_selection(moe_lib):
    c = np.zeros((3, 8), np.int32)
    c[:, :4] = 5
    _indices(moe_lib, c, 4, 2, 2, 6)
    _indices(moe_lib, c, 4, 2, 2, 0)


def _combine(moe, src, coeff, idx, G):
    n, H = src.shape
    print(f"dered combine n={n} H={H} G={G} coeff={coeff is not None}", flush=True)
    wb = moe.dered_combine_alloc(to_dev_bf16(src), to_dev(coeff) if coeff is not None else None,
                                 to_dev(idx), G)
    torch.cuda.synchronize()
    ref, _ = oracle.scatter_add_rows(src, idx, G, coeff)
    np.testing.assert_array_equal(bits(wb), ref)


@pytest.mark.parametrize("oep,E,iep,El,start,H,seed", [
    (4, 16, 2, 4, 4, 8, 6), (8, 64, 4, 8, 32, 136, 7), (2, 300, 3, 7, 100, 1032, 8),
])
def test_dered_combine_random(moe_lib, oep, E, iep, El, start, H, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 20, size=(oep, E)).astype(np.int32)
    idx, _, tot = oracle.dered_indices(c, start, iep, El)
    G = int(c.sum())
    src = W.normal_bf16(rng, (tot, H))
    coeff = rng.standard_normal(tot).astype(np.float32)
    _combine(moe_lib, src, coeff, idx[:tot], G)
    _combine(moe_lib, src, None, idx[:tot], G)
    # indices past G are skipped
    bad = idx[:tot].copy()
    bad[::5] = G + 3
    _combine(moe_lib, src, coeff, bad, G)


def test_dered_combine_signed_zeros(moe_lib):
    """zeros + (-0) is +0: a zero value or coefficient gives +0, with or without
    coefficients; a nonzero product keeps its sign."""
    rng = np.random.default_rng(10)
    n, H, G = 64, 16, 80
    src = W.normal_bf16(rng, (n, H))
    src[::3, ::2] = 0x8000                                  # -0
    src[1::3, 1::2] = 0x0000
    coeff = rng.standard_normal(n).astype(np.float32)
    coeff[5] = 0.0
    coeff[6] = -0.0
    idx = rng.permutation(G)[:n].astype(np.int32)
    _combine(moe_lib, src, coeff, idx, G)
    _combine(moe_lib, src, None, idx, G)


def test_dered_workload_end_to_end(moe_lib):
    """Eight sources x 256 experts, 65,536 gathered rows of H=2048: the device
    indices feed the device whiteboard combine."""
    d = W.gen_dered()
    c = d["cfg"]
    got, idx, tot = _indices(moe_lib, d["counts"], c["expert_start"], c["iep"], c["El"],
                             d["n_selected"])
    wb = moe_lib.dered_combine_alloc(to_dev_bf16(d["outer_output"]), to_dev(d["router_coeff"]),
                                     got["indices"], d["G"])
    torch.cuda.synchronize()
    ref, _ = oracle.scatter_add_rows(d["outer_output"], idx, d["G"], d["router_coeff"])
    np.testing.assert_array_equal(bits(wb), ref)


def _combine_dup(moe, src, coeff, idx, G):
    """Whiteboard with repeated indices: rows with one source bit-exact, rows
    with several within 1e-2 of the fp64 sum; two runs give the same bits."""
    n, H = src.shape
    G_ok = (idx >= 0) & (idx < G)
    mult = np.bincount(idx[G_ok], minlength=G)
    print(f"dered combine n={n} H={H} G={G} max sources per row {mult.max()}", flush=True)
    args = (to_dev_bf16(src), to_dev(coeff) if coeff is not None else None, to_dev(idx))
    wb1 = bits(moe.dered_combine_alloc(*args, G))
    wb2 = bits(moe.dered_combine_alloc(*args, G))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wb1, wb2)
    ref, ref64 = oracle.scatter_add_rows(src, idx, G, coeff)
    single = mult <= 1
    np.testing.assert_array_equal(wb1[single], ref[single])
    assert_rel(f64(wb1[~single]), ref64[~single], 1e-2, "rows with several sources")


def test_dered_combine_duplicates(moe_lib):
    rng = np.random.default_rng(11)
    n, G, H = 600, 150, 136                      # ~4 sources per row, H/8 = 17 chunks
    src = W.normal_bf16(rng, (n, H))
    idx = rng.integers(0, G, size=n).astype(np.int32)
    idx[::37] = G + 2                            # skipped
    idx[::41] = -1                               # skipped
    coeff = rng.standard_normal(n).astype(np.float32)
    _combine_dup(moe_lib, src, coeff, idx, G)
    _combine_dup(moe_lib, src, None, idx, G)


def test_dered_combine_long_segment(moe_lib):
    """One row named by 200 sources (more than a wave's lanes), the others by
    at most one; H = 2064 takes the row in several passes of the wave."""
    rng = np.random.default_rng(12)
    n, G, H = 260, 80, 2064
    src = W.normal_bf16(rng, (n, H))
    idx = np.concatenate([np.full(200, 7), rng.permutation(np.delete(np.arange(G), 7))[:60]])
    idx = rng.permutation(idx).astype(np.int32)
    coeff = rng.uniform(0.5, 1.5, n).astype(np.float32)
    _combine_dup(moe_lib, src, coeff, idx, G)


def test_dered_combine_many_rows(moe_lib):
    """More rows than the one-workgroup scan takes (65,536): the three-kernel
    scan of the per-row counts, with repeated and out-of-range indices."""
    rng = np.random.default_rng(13)
    n, G, H = 3000, 70_001, 8
    src = W.normal_bf16(rng, (n, H))
    idx = rng.integers(0, G, size=n).astype(np.int32)
    idx[:40] = idx[40:80]                        # 40 rows named twice
    idx[100] = G                                 # skipped
    coeff = rng.standard_normal(n).astype(np.float32)
    _combine_dup(moe_lib, src, coeff, idx, G)
