"""Shared test utilities: host <-> device transfers of bf16 bit arrays and the
tolerance rules of the parity tests."""
from __future__ import annotations

import numpy as np
import torch

import moe_workloads as W


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)) \
        .view(torch.bfloat16).to(dev())


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(bits_arr: np.ndarray) -> np.ndarray:
    return W.f32_from_bf16(bits_arr).astype(np.float64)


def assert_rel(got: np.ndarray, ref: np.ndarray, rel: float = 1e-2, what: str = ""):
    """Elementwise |got - ref| <= rel*|ref| + rel*rms(ref), rms over the whole tensor
    (the second term covers elements that are near zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + rel * rms
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {ref.size} elements outside the "
                           f"{rel} relative bound; worst err {err.max():.3e} (rms {rms:.3e})")


def gemm_tol(H: int) -> float:
    """Max-abs bound of the grouped GEMM against the fp64 oracle: 2e-2 * sqrt(H) / 64."""
    return 2e-2 * np.sqrt(H) / 64.0


def ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> int:
    """Largest distance in bf16 units in the last place (sign-magnitude ordering)."""
    def key(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    if a_bits.size == 0:
        return 0
    return int(np.max(np.abs(key(a_bits) - key(b_bits))))


def assert_h_within_ulp(h_bits: np.ndarray, h_ref: np.ndarray, what: str = "h"):
    """h is stored as bf16: it must sit within one bf16 ulp (2^-8 relative) of
    the fp64 value, plus a small absolute term for the fp32 accumulation of
    g and u."""
    got = f64(h_bits)
    rms = float(np.sqrt(np.mean(h_ref ** 2))) if h_ref.size else 0.0
    err = np.abs(got - h_ref)
    bound = 2.0 ** -8 * np.abs(h_ref) + 1e-4 * rms
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond one bf16 ulp; worst {err.max():.3e}"


BF16_U = 2.0 ** -8   # unit roundoff of bf16 (8-bit significand, round to nearest)


def assert_dot_bound(got, ref, terms, what="", term_units=4, out_units=2):
    """Elementwise error bound of a sum of products whose inputs went through
    bf16: |got - ref| <= term_units * u * T + out_units * u * |ref|, with T the
    sum of the magnitudes of the exact terms and u = 2^-8. Two roundings of an
    input term (an intermediate stored as bf16 from a bf16-rounded operand)
    cost at most 2u * T, the bf16 output u * |ref|; the bound doubles both."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape == np.shape(terms), (got.shape, ref.shape, np.shape(terms))
    bound = term_units * BF16_U * np.asarray(terms) + out_units * BF16_U * np.abs(ref)
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {ref.size} elements outside the bf16 "
                           f"dot-product bound; worst err/bound {float(np.max(err / (bound + 1e-300))):.3f}")
    return float(np.max(err / (bound + 1e-300))) if ref.size else 0.0


def ffn_grad_worst(got, ref, x, off, wg, wu, wd, dy, h64, experts):
    """Checks the grouped SwiGLU FFN backward of the given experts against the
    oracle's fp64 result with assert_dot_bound: dx rows of each expert and its
    three weight gradients. The magnitudes of the exact terms come from the
    oracle's intermediates (|dg|, |du|, the forward's fp64 h). Returns the worst
    err/bound ratio per output."""
    f = lambda b: np.abs(f64(b))
    worst = dict(dx=0.0, dw_gate=0.0, dw_up=0.0, dw_down=0.0)
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        dg, du = np.abs(ref["dg"][lo:hi]), np.abs(ref["du"][lo:hi])
        X = f(x[lo:hi])
        pairs = (("dx", got["dx"][lo:hi], ref["dx"][lo:hi],
                  lambda: dg @ f(wg[e]).T + du @ f(wu[e]).T),
                 ("dw_gate", got["dw_gate"][e], ref["dwg"][e], lambda: X.T @ dg),
                 ("dw_up", got["dw_up"][e], ref["dwu"][e], lambda: X.T @ du),
                 ("dw_down", got["dw_down"][e], ref["dwd"][e],
                  lambda: np.abs(h64[lo:hi]).T @ f(dy[lo:hi])))
        for name, g, r, terms in pairs:
            worst[name] = max(worst[name], assert_dot_bound(g, r, terms(), f"{name} expert {e}"))
    return worst
