"""Pins of the oracle's bf16 codec against torch's float32->bfloat16 conversion
(a library routine, round to nearest even) and hand-worked rounding cases."""
import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_encode_matches_torch_on_fp32_values():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # fp32 subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        # exact bf16 ties: bf16 value plus half an ulp
        ((rng.integers(0, 2**15, 20000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    vals = vals[np.isfinite(vals)]
    got = oracle.f64_to_bf16(vals.astype(np.float64))
    np.testing.assert_array_equal(got, _torch_bf16_bits(vals))


def test_roundtrip_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    finite = bits[exp != 0xFF]
    dec = oracle.bf16_to_f64(finite)
    np.testing.assert_array_equal(oracle.f64_to_bf16(dec), finite)


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2**-8, 0x3F80),             # tie between 0x3F80 and 0x3F81 -> even
    (1.0 + 3 * 2**-8, 0x3F82),         # tie between 0x3F81 and 0x3F82 -> even
    (1.0 + 2**-8 + 2**-40, 0x3F81),    # just above the tie: an fp32 detour would give 0x3F80
    (1.0 + 2**-8 - 2**-40, 0x3F80),
    (-(1.0 + 2**-8 + 2**-40), 0xBF81),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (2.0**-133, 0x0001),               # smallest subnormal
    (2.0**-134, 0x0000),               # tie between 0 and the smallest subnormal -> even
    (1.5 * 2.0**-134, 0x0001),
    (2.0**-126, 0x0080),               # smallest normal
    (127.5 * 2.0**-133, 0x0080),       # subnormal tie rounding up into the smallest normal
    (3.3895313892515355e38, 0x7F7F),   # largest finite
    (3.4e38, 0x7F80),                  # rounds past the largest finite
])
def test_hand_worked_rounding(value, bits):
    assert oracle.f64_to_bf16_scalar(value) == bits
