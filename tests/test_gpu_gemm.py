"""GPU parity of moe_grouped_gemm_swiglu against the fp64 oracle: max-abs
error of y (and h) within 2e-2 * sqrt(H) / 64."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_h_within_ulp, bits, f64, gemm_tol, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _gemm(moe, x, off, wg, wu, wd):
    E, H, I = wg.shape
    print(f"gemm N={x.shape[0]} E={E} H={H} I={I} rows={int(off[-1])}", flush=True)
    h, y = moe.grouped_gemm_alloc(to_dev_bf16(x), to_dev(off), to_dev_bf16(wg), to_dev_bf16(wu),
                                  to_dev_bf16(wd))
    torch.cuda.synchronize()
    return bits(h), bits(y)


@pytest.mark.parametrize("counts,H,I,seed", [
    ([1], 64, 64, 0),
    ([5, 0, 130, 1, 0, 64], 128, 64, 1),          # empty experts, ragged tiles
    ([300, 2, 0, 129], 320, 192, 2),              # H not a multiple of 256, I of 128
    ([1000, 17, 256, 3, 0, 0, 513], 512, 256, 3),
    ([0, 0, 0], 64, 128, 4),                      # no rows at all
])
def test_gemm_small(moe_lib, counts, H, I, seed):
    rng = np.random.default_rng(seed)
    E = len(counts)
    off = _offsets(counts)
    N = int(off[-1]) + 3                           # capacity rows past the last expert
    x = W.normal_bf16(rng, (N, H))
    # the weight scale of the workloads, N(0, 0.02^2): the y bound is stated for it
    wg = W.normal_bf16(rng, (E, H, I), 0.02)
    wu = W.normal_bf16(rng, (E, H, I), 0.02)
    wd = W.normal_bf16(rng, (E, I, H), 0.02)
    hb, yb = _gemm(moe_lib, x, off, wg, wu, wd)
    n = int(off[-1])
    if n == 0:
        return
    h_ref, y_ref = oracle.grouped_swiglu(x[:n], off, wg, wu, wd)
    assert np.max(np.abs(f64(yb[:n]) - y_ref)) <= gemm_tol(H)
    assert_h_within_ulp(hb[:n], h_ref)


def _many_expert_counts(seed, E=1000, busy=40):
    """E experts, most of them empty; `busy` of them (the last one included)
    with 1..300 rows."""
    rng = np.random.default_rng(seed)
    counts = np.zeros(E, np.int64)
    sel = np.concatenate([rng.choice(E - 1, busy - 1, replace=False), [E - 1]])
    counts[sel] = rng.integers(1, 301, size=busy)
    return counts


def test_gemm_many_experts(moe_lib):
    # E = 1000 (not a multiple of 16): the tile lookup's last expert block is
    # partial, and most experts have no rows
    counts = _many_expert_counts(31)
    rng = np.random.default_rng(32)
    E, H, I = len(counts), 64, 64
    off = _offsets(counts)
    N = int(off[-1]) + 5
    x = W.normal_bf16(rng, (N, H))
    wg = W.normal_bf16(rng, (E, H, I), 0.02)
    wu = W.normal_bf16(rng, (E, H, I), 0.02)
    wd = W.normal_bf16(rng, (E, I, H), 0.02)
    hb, yb = _gemm(moe_lib, x, off, wg, wu, wd)
    n = int(off[-1])
    h_ref, y_ref = oracle.grouped_swiglu(x[:n], off, wg, wu, wd)
    assert np.max(np.abs(f64(yb[:n]) - y_ref)) <= gemm_tol(H)
    assert_h_within_ulp(hb[:n], h_ref)


@pytest.mark.parametrize("H,I,rows_per_expert,seed", [
    (64, 64, 12_345, 41),    # one k-step per tile in both passes
    (128, 128, 6_001, 42),   # two k-steps per tile
])
def test_gemm_many_tiles_short_k(moe_lib, H, I, rows_per_expert, seed):
    # several tiles per workgroup with tiles of one or two k-steps: the loads
    # that run ahead cross tile boundaries and a workgroup's two load-free
    # k-steps fall into different tiles
    rng = np.random.default_rng(seed)
    counts = [rows_per_expert] * 7 + [rows_per_expert // 3]
    E = len(counts)
    off = _offsets(counts)
    N = int(off[-1]) + 7
    x = W.normal_bf16(rng, (N, H))
    wg = W.normal_bf16(rng, (E, H, I), 0.02)
    wu = W.normal_bf16(rng, (E, H, I), 0.02)
    wd = W.normal_bf16(rng, (E, I, H), 0.02)
    hb, yb = _gemm(moe_lib, x, off, wg, wu, wd)
    n = int(off[-1])
    h_ref, y_ref = oracle.grouped_swiglu(x[:n], off, wg, wu, wd)
    assert np.max(np.abs(f64(yb[:n]) - y_ref)) <= gemm_tol(H)
    assert_h_within_ulp(hb[:n], h_ref)


def test_gemm_config1(moe_lib):
    g = W.gen_c1()
    c = g["cfg"]
    p = oracle.permute(g["x"], g["expert_ids"], c["E"])
    hb, yb = _gemm(moe_lib, p["permuted"], p["expert_offsets"], g["w_gate"], g["w_up"],
                   g["w_down"])
    h_ref, y_ref = oracle.grouped_swiglu(p["permuted"], p["expert_offsets"], g["w_gate"],
                                         g["w_up"], g["w_down"])
    tol = gemm_tol(c["H"])
    err = np.max(np.abs(f64(yb) - y_ref))
    print(f"config 1: max |y - ref| = {err:.3e} (bound {tol:.3e})")
    assert err <= tol
    assert_h_within_ulp(hb, h_ref)

