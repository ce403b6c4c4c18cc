"""GPU parity of moe_unpermute_grad: d_permuted bit-exact (correctly rounded
product on both sides), d_probs within the 1e-2 relative bound."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_rel, bits, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run(moe, g, perm, ros, probs):
    T, K = probs.shape
    print(f"grad T={T} K={K} N={perm.shape[0]} H={perm.shape[1]}", flush=True)
    init = torch.zeros(perm.shape, dtype=torch.bfloat16, device="cuda")
    dp, dpr = moe.unpermute_grad_alloc(to_dev_bf16(g), to_dev_bf16(perm), to_dev(ros),
                                       to_dev(probs), d_permuted=init)
    torch.cuda.synchronize()
    rdp, rdpr, _, rdpr64 = oracle.unpermute_grad(g, perm, ros, probs)
    np.testing.assert_array_equal(bits(dp), rdp)
    assert_rel(dpr.cpu().numpy(), rdpr64, 1e-2, "d_probs")


# Kernel instance reached (16-byte chunks per lane, waves per token): rows of
# at least 2048 elements below 32,768 tokens take two waves per token.
@pytest.mark.parametrize("T,K,E,H,seed", [
    (1, 1, 1, 8, 0), (300, 2, 8, 128, 1), (1000, 6, 64, 264, 2),   # 1 chunk, 1 wave
    (300, 2, 8, 1000, 6),          # 2 chunks, 1 wave
    (257, 4, 16, 1536, 7),         # 4 chunks, 1 wave (3 used)
    (8192, 2, 64, 2048, 11),       # 2 chunks, 2 waves (the skewed layer's shape)
    (513, 8, 32, 4096, 3),         # 4 chunks, 2 waves
    (200, 3, 16, 6144, 8),         # 8 chunks, 2 waves (6 used)
    (32768, 1, 4, 2056, 9),        # 8 chunks, 1 wave (5 used)
    (32768, 1, 4, 4104, 10),       # 16 chunks, 1 wave (9 used)
    (64, 16, 20, 8200, 4),         # 16 chunks, 2 waves (9 used)
])
def test_grad_random(moe_lib, T, K, E, H, seed):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ros = oracle.permute(None, ids, E, rows=False)["row_of_slot"]
    probs = rng.standard_normal((T, K)).astype(np.float32)
    _run(moe_lib, W.normal_bf16(rng, (T, H)), W.normal_bf16(rng, (T * K, H)), ros, probs)


def test_grad_dropped_slots(moe_lib):
    rng = np.random.default_rng(5)
    T, K, E, H = 200, 4, 10, 64
    ids = rng.integers(0, E + 3, size=(T, K)).astype(np.int32)
    ros = oracle.permute(None, ids, E, rows=False)["row_of_slot"]
    _run(moe_lib, W.normal_bf16(rng, (T, H)), W.normal_bf16(rng, (T * K, H)), ros,
         rng.random((T, K)).astype(np.float32))


def _tie_cases(n):
    """(p, g) pairs whose fp32 product lands exactly on a bf16 midpoint while the
    exact product does not: a one-step fp32 rounding would then round wrongly half
    of the time."""
    rng = np.random.default_rng(7)
    ps, gs = [], []
    while len(ps) < n:
        gb = np.uint16(rng.integers(0x3F81, 0x4000))
        g = float(W.f32_from_bf16(np.array([gb]))[0])
        mid = np.array([(int(rng.integers(0x3F80, 0x407F)) << 16) | 0x8000], np.uint32)
        m = float(mid.view(np.float32)[0])
        p0 = np.float32(m / g)
        for d in (-2, -1, 0, 1, 2):
            p = np.float32(p0 + d * np.spacing(p0))
            r = np.float32(p) * np.float32(g)
            if (int(np.array([r]).view(np.uint32)[0]) & 0xFFFF) == 0x8000 and \
                    float(p) * g != float(r):
                sgn = 1.0 if rng.random() < 0.5 else -1.0
                ps.append(np.float32(sgn * p))
                gs.append(gb)
                break
    return np.array(ps, np.float32), np.array(gs, np.uint16)


def test_grad_ties_round_correctly(moe_lib):
    T, H = 256, 8
    p, gb = _tie_cases(T)
    g = np.repeat(gb[:, None], H, axis=1)
    ros = np.arange(T, dtype=np.int32).reshape(T, 1)
    # the exact products differ from a plain RNE of the fp32 product for many rows
    exact = oracle.f64_to_bf16(p.astype(np.float64) * W.f32_from_bf16(gb).astype(np.float64))
    naive = W.bf16_from_f32(p * W.f32_from_bf16(gb))
    assert int((exact != naive).sum()) > T // 4
    _run(moe_lib, g, W.normal_bf16(np.random.default_rng(0), (T, H)), ros, p.reshape(T, 1))


def test_grad_config5(moe_lib):
    g = W.gen_c5()
    c = g["cfg"]
    ros = oracle.permute(None, g["expert_ids"], c["E"], rows=False)["row_of_slot"]
    _run(moe_lib, g["grad_out"], g["permuted"], ros, g["probs"])
