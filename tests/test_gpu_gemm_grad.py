"""GPU parity of moe_grouped_gemm_swiglu_grad (the grouped SwiGLU FFN backward)
against the fp64 oracle. The GPU takes h as its forward stored it (bf16) and
keeps dh and [dg | du] as bf16 between its GEMMs, so each output element is a
sum of terms that went through up to two bf16 roundings: every element is
checked against the dot-product bound |err| <= 4u * sum|terms| + 2u * |ref|
(u = 2^-8, the terms from the oracle's exact intermediates), twice the worst
case of that arithmetic."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_dot_bound, bits, f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _gpu(moe, x, off, wg, wu, wd, dy):
    E, H, I = wg.shape
    print(f"gemm grad N={x.shape[0]} E={E} H={H} I={I} rows={int(off[-1])}", flush=True)
    xd, od = to_dev_bf16(x), to_dev(off)
    wgd, wud, wdd = to_dev_bf16(wg), to_dev_bf16(wu), to_dev_bf16(wd)
    h, _ = moe.grouped_gemm_alloc(xd, od, wgd, wud, wdd)
    g = moe.grouped_gemm_grad_alloc(xd, od, wgd, wud, wdd, h, to_dev_bf16(dy))
    torch.cuda.synchronize()
    return {k: f64(bits(v)) for k, v in g.items()}


def _terms(x, off, wg, wu, wd, dy, ref, experts):
    """Sum of the magnitudes of the exact terms of every checked element."""
    f = lambda b: np.abs(f64(b))
    h, _ = oracle.grouped_swiglu(x, off, wg, wu, wd)
    T = {}
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        dg, du = np.abs(ref["dg"][lo:hi]), np.abs(ref["du"][lo:hi])
        X = f(x[lo:hi])
        T[e] = dict(dx=dg @ f(wg[e]).T + du @ f(wu[e]).T, dwg=X.T @ dg, dwu=X.T @ du,
                    dwd=np.abs(h[lo:hi]).T @ f(dy[lo:hi]))
    return T


def _check(got, ref, x, off, wg, wu, wd, dy, experts=None):
    E = len(off) - 1
    experts = range(E) if experts is None else experts
    T = _terms(x, off, wg, wu, wd, dy, ref, experts)
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        t = T[e]
        assert_dot_bound(got["dx"][lo:hi], ref["dx"][lo:hi], t["dx"], f"dx expert {e}")
        assert_dot_bound(got["dw_gate"][e], ref["dwg"][e], t["dwg"], f"dw_gate expert {e}")
        assert_dot_bound(got["dw_up"][e], ref["dwu"][e], t["dwu"], f"dw_up expert {e}")
        assert_dot_bound(got["dw_down"][e], ref["dwd"][e], t["dwd"], f"dw_down expert {e}")


def _data(seed, counts, H, I, pad=3):
    rng = np.random.default_rng(seed)
    E = len(counts)
    off = _offsets(counts)
    N = int(off[-1]) + pad
    x = W.normal_bf16(rng, (N, H))
    wg = W.normal_bf16(rng, (E, H, I), 0.02)
    wu = W.normal_bf16(rng, (E, H, I), 0.02)
    wd = W.normal_bf16(rng, (E, I, H), 0.02)
    dy = W.normal_bf16(rng, (N, H))
    return x, off, wg, wu, wd, dy


@pytest.mark.parametrize("counts,H,I,seed", [
    ([1], 64, 64, 0),
    ([5, 0, 130, 1, 0, 64], 128, 64, 1),          # empty experts, ragged tiles, I < 128
    ([300, 2, 0, 129], 320, 192, 2),              # H and I not multiples of 128
    ([1000, 17, 256, 3, 0, 0, 513], 512, 256, 3),
    ([0, 0, 0], 64, 128, 4),                      # no rows: zero weight gradients
])
def test_gemm_grad_small(moe_lib, counts, H, I, seed):
    x, off, wg, wu, wd, dy = _data(seed, counts, H, I)
    got = _gpu(moe_lib, x, off, wg, wu, wd, dy)
    ref = oracle.grouped_swiglu_grad(x, off, wg, wu, wd, dy)
    _check(got, ref, x, off, wg, wu, wd, dy)
    assert not np.any(got["dx"][int(off[-1]):])    # rows past the experts are not written
    for e, c in enumerate(counts):
        if c == 0:
            assert not got["dw_gate"][e].any() and not got["dw_down"][e].any()


def test_gemm_grad_many_experts(moe_lib):
    # E = 1000, most experts empty (their weight gradients must be zero)
    rng = np.random.default_rng(41)
    E = 1000
    counts = np.zeros(E, np.int64)
    sel = np.concatenate([rng.choice(E - 1, 29, replace=False), [E - 1]])
    counts[sel] = rng.integers(1, 201, size=30)
    x, off, wg, wu, wd, dy = _data(42, counts, 64, 64)
    got = _gpu(moe_lib, x, off, wg, wu, wd, dy)
    ref = oracle.grouped_swiglu_grad(x, off, wg, wu, wd, dy)
    _check(got, ref, x, off, wg, wu, wd, dy)
    empty = counts == 0
    assert not got["dw_gate"][empty].any() and not got["dw_up"][empty].any()
    assert not got["dw_down"][empty].any()


def test_gemm_grad_config1(moe_lib):
    g = W.gen_c1()
    c = g["cfg"]
    p = oracle.permute(g["x"], g["expert_ids"], c["E"])
    dy = W.normal_bf16(np.random.default_rng(11), p["permuted"].shape)
    got = _gpu(moe_lib, p["permuted"], p["expert_offsets"], g["w_gate"], g["w_up"], g["w_down"], dy)
    ref = oracle.grouped_swiglu_grad(p["permuted"], p["expert_offsets"], g["w_gate"], g["w_up"],
                                     g["w_down"], dy)
    _check(got, ref, p["permuted"], p["expert_offsets"], g["w_gate"], g["w_up"], g["w_down"], dy)



@pytest.mark.parametrize("counts,H,I,seed", [
    ([5, 0, 130, 1, 0, 64], 128, 64, 21),
    ([300, 2, 0, 129], 320, 192, 22),
    ([0, 0, 0], 64, 128, 23),
])
def test_gemm_saved_preact(moe_lib, counts, H, I, seed):
    """The forward's optional pre-activations: g and u in fp32 as the SwiGLU
    used them (against fp64 x.W within the fp32 accumulation bound), h and y
    unchanged by keeping them, and a backward from them that gives the same
    bits as the one that recomputes them."""
    x, off, wg, wu, wd, dy = _data(seed, counts, H, I)
    E = len(counts)
    n = int(off[-1])
    print(f"saved pre-activations N={x.shape[0]} E={E} H={H} I={I} rows={n}", flush=True)
    xd, od = to_dev_bf16(x), to_dev(off)
    wgd, wud, wdd = to_dev_bf16(wg), to_dev_bf16(wu), to_dev_bf16(wd)
    h0, y0 = moe_lib.grouped_gemm_alloc(xd, od, wgd, wud, wdd)
    h1, y1, pre = moe_lib.grouped_gemm_alloc(xd, od, wgd, wud, wdd, keep_preact=True)
    dyd = to_dev_bf16(dy)
    g0 = moe_lib.grouped_gemm_grad_alloc(xd, od, wgd, wud, wdd, h0, dyd)
    g1 = moe_lib.grouped_gemm_grad_alloc(xd, od, wgd, wud, wdd, h0, dyd, preact=pre)
    torch.cuda.synchronize()
    assert torch.equal(h0[:n], h1[:n]) and torch.equal(y0[:n], y1[:n])
    for k in g0:
        a, b = (g0[k][:n], g1[k][:n]) if k == "dx" else (g0[k], g1[k])
        assert torch.equal(a, b), k
    P = pre.cpu().numpy().astype(np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if lo == hi:
            continue
        X = f64(x[lo:hi])
        for j, w in ((0, wg[e]), (1, wu[e])):
            ref = X @ f64(w)
            bound = 2.0 ** -13 * (np.abs(X) @ np.abs(f64(w))) + 1e-30
            err = np.abs(P[lo:hi, j * I:(j + 1) * I] - ref)
            assert np.all(err <= bound), f"expert {e} {'gu'[j]}: worst err/bound {np.max(err / bound):.3f}"
