"""GPU parity of x_active_mask (a [T] token mask or a [T, K] slot mask; a slot
outside it is not dispatched) in moe_permute, moe_unpermute_combine and
moe_unpermute_combine_grad, against the oracle: indices and rows bit-exact,
combine outputs and gradients within the 1e-2 relative bound."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_rel, bits, f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _masks(rng, T, K):
    n = int(rng.integers(0, T + 1))
    return {
        "prefix": np.arange(T) < n,                    # the page's form: trues first
        "tokens": rng.random(T) < 0.7,                 # any pattern, applied flag by flag
        "slots": rng.random((T, K)) < 0.7,
        "none_active": np.zeros((T, K), bool),
    }


def _dev_mask(m):
    return torch.from_numpy(np.ascontiguousarray(m)).to("cuda")


@pytest.mark.parametrize("T,K,E,H,seed", [(1, 1, 2, 8, 0), (700, 6, 64, 136, 1),
                                          (3000, 8, 256, 64, 2), (4097, 16, 40, 16, 3)])
def test_masked_permute(moe_lib, T, K, E, H, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, E + 2, size=(T, K)).astype(np.int32)
    x = W.normal_bf16(rng, (T, H))
    for name, m in _masks(rng, T, K).items():
        print(f"masked permute {name} T={T} K={K} E={E} H={H}", flush=True)
        got = moe_lib.permute_alloc(to_dev_bf16(x), to_dev(ids), E, active_mask=_dev_mask(m))
        torch.cuda.synchronize()
        ref = oracle.permute(x, ids, E, active_mask=m)
        for key in ("expert_counts", "expert_offsets", "sorted_slot", "row_of_slot"):
            np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
        n = int(ref["expert_offsets"][-1])
        np.testing.assert_array_equal(bits(got["permuted"][:n]), ref["permuted"][:n])


def test_masked_combine_and_backward(moe_lib):
    """The masked permute's rows, combined and differentiated under the same mask,
    with zero / copy / const experts and a shared term."""
    rng = np.random.default_rng(9)
    T, K, E, H, Z, C, NC = 900, 6, 24, 264, 2, 2, 2
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    sp_slots = rng.random((T, K)) < 0.25
    ids[sp_slots] = E + rng.integers(0, Z + C + NC, size=int(sp_slots.sum()))
    probs = rng.standard_normal((T, K)).astype(np.float32)
    x, g = W.normal_bf16(rng, (T, H)), W.normal_bf16(rng, (T, H))
    ori, shared = W.normal_bf16(rng, (T, H)), W.normal_bf16(rng, (T, H))
    cv = W.normal_bf16(rng, (NC, H))
    a1 = rng.uniform(-1, 1, T).astype(np.float32)
    a2 = rng.uniform(-1, 1, T).astype(np.float32)
    keep = [to_dev_bf16(ori), to_dev(a1), to_dev(a2), to_dev_bf16(cv)]
    sp = moe_lib.make_special(Z, C, NC, keep[0], keep[1], keep[2], (1, 0, 0), keep[3])
    kw = dict(num_zero=Z, num_copy=C, num_const=NC, ori_x=ori, alpha1=a1, alpha2=a2,
              alpha_strides=(1, 0, 0), const_v=cv)
    for name, m in _masks(rng, T, K).items():
        print(f"masked combine {name} T={T} K={K} E={E} H={H}", flush=True)
        dm = _dev_mask(m)
        p = moe_lib.permute_alloc(to_dev_bf16(x), to_dev(ids), E, active_mask=dm)
        out = moe_lib.combine_alloc(p["permuted"], p["row_of_slot"], to_dev(ids), to_dev(probs),
                                    E, special=sp, shared_x=to_dev_bf16(shared), active_mask=dm)
        gr = moe_lib.combine_grad_alloc(to_dev_bf16(g), p["permuted"], p["row_of_slot"],
                                        to_dev(ids), to_dev(probs), E, special=sp,
                                        alpha_numel=T, active_mask=dm)
        torch.cuda.synchronize()
        ref_p = oracle.permute(x, ids, E, active_mask=m)
        _, ref64 = oracle.combine(ref_p["permuted"], ref_p["row_of_slot"], ids, probs, E,
                                  shared_x=shared, active_mask=m, **kw)
        assert_rel(f64(bits(out)), ref64, 1e-2, f"combine {name}")
        if name == "none_active":
            np.testing.assert_array_equal(bits(out), shared)
        rg = oracle.combine_grad(g, ref_p["permuted"], ref_p["row_of_slot"], ids, probs, E,
                                 active_mask=m, **kw)
        assert_rel(gr["d_probs"].cpu().numpy(), rg["d_probs"], 1e-2, f"d_probs {name}")
        slot_mask = m if m.ndim == 2 else np.repeat(m[:, None], K, 1)
        assert not np.any(gr["d_probs"].cpu().numpy()[~slot_mask]), "masked slots: d_probs = 0"
        assert_rel(f64(bits(gr["d_ori_x"])), rg["d_ori_x"], 1e-2, f"d_ori_x {name}")
        assert_rel(f64(bits(gr["d_const_v"])), rg["d_const_v"], 1e-2, f"d_const_v {name}")
        assert_rel(gr["d_alpha1"].cpu().numpy(), rg["d_alpha1"], 1e-2, f"d_alpha1 {name}")
        w = rg["row_written"]
        np.testing.assert_array_equal(bits(gr["d_expert_out"])[w],
                                      oracle.f64_to_bf16(rg["d_expert_out"][w]))


def test_mask_shape_is_checked(moe_lib):
    ids = torch.zeros((8, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        moe_lib.permute_alloc(None, ids, 4, rows=False,
                              active_mask=torch.ones(7, dtype=torch.bool, device="cuda"))
