"""GPU parity of moe_unpermute_combine against the oracle: exact round trips,
the 1e-2 relative bound elsewhere (fp32 accumulation, bf16 output)."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_rel, bits, f64, to_dev, to_dev_bf16, ulp_diff

pytestmark = pytest.mark.gpu


def _special(moe, Z, C, Nc, ori=None, a1=None, a2=None, strides=(0, 0, 0), cv=None):
    keep = [to_dev_bf16(ori) if ori is not None else None,
            to_dev(a1) if a1 is not None else None,
            to_dev(a2) if a2 is not None else None,
            to_dev_bf16(cv) if cv is not None else None]
    sp = moe.make_special(Z, C, Nc, keep[0], keep[1], keep[2], strides, keep[3])
    return sp, keep


def _combine_both(moe, eo, ros, ids, probs, E, *, row_map=None, Z=0, C=0, Nc=0, ori=None,
                  a1=None, a2=None, strides=(0, 0, 0), cv=None, shared=None):
    T, K = ids.shape
    print(f"combine T={T} K={K} E={E} H={eo.shape[1]} special={Z},{C},{Nc}", flush=True)
    sp, keep = _special(moe, Z, C, Nc, ori, a1, a2, strides, cv) if (Z + C + Nc) else (None, [])
    got = moe.combine_alloc(to_dev_bf16(eo), to_dev(ros), to_dev(ids), to_dev(probs), E,
                            row_map=to_dev(row_map) if row_map is not None else None, special=sp,
                            shared_x=to_dev_bf16(shared) if shared is not None else None)
    torch.cuda.synchronize()
    ref, ref64 = oracle.combine(eo, ros, ids, probs, E, row_map=row_map, num_zero=Z, num_copy=C,
                                num_const=Nc, ori_x=ori, alpha1=a1, alpha2=a2,
                                alpha_strides=strides, const_v=cv, shared_x=shared)
    return bits(got), ref, ref64


@pytest.mark.parametrize("T,E,H", [(1, 1, 8), (333, 7, 136), (2048, 64, 2048),
                                   (901, 24, 2120)])  # 4 waves per token, 265 chunks: uneven parts
def test_top1_roundtrip_bit_exact(moe_lib, T, E, H):
    rng = np.random.default_rng(T)
    x = W.normal_bf16(rng, (T, H))
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    p = moe_lib.permute_alloc(to_dev_bf16(x), to_dev(ids), E)
    out = moe_lib.combine_alloc(p["permuted"], p["row_of_slot"], to_dev(ids),
                                torch.ones((T, 1), dtype=torch.float32, device="cuda"), E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), x)


@pytest.mark.parametrize("K", [2, 6, 16])
def test_topk_unit_probs_bit_exact(moe_lib, K):
    rng = np.random.default_rng(K)
    T, E, H = 700, 32, 264
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    got, ref, _ = _combine_both(moe_lib, p["permuted"], p["row_of_slot"], ids,
                                np.ones((T, K), np.float32), E)
    np.testing.assert_array_equal(got, ref)   # K*x exact in fp32 -> same rounding


@pytest.mark.parametrize("cfg", [1, 2])
def test_combine_configs(moe_lib, cfg):
    g = W.generate(cfg, **({"with_weights": False} if cfg == 1 else {}))
    E = g["cfg"]["E"]
    p = oracle.permute(g["x"], g["expert_ids"], E)
    got, ref, ref64 = _combine_both(moe_lib, p["permuted"], p["row_of_slot"], g["expert_ids"],
                                    g["probs"], E)
    assert_rel(f64(got), ref64, 1e-2, "combine")
    assert ulp_diff(got, ref) <= 1


def test_combine_special_experts_and_shared(moe_lib):
    rng = np.random.default_rng(21)
    T, K, E, H, Z, C, Nc = 1500, 8, 16, 520, 3, 2, 4
    ids = rng.integers(0, E + Z + C + Nc + 2, size=(T, K)).astype(np.int32)  # some dropped
    x = W.normal_bf16(rng, (T, H))
    p = oracle.permute(x, ids, E)
    eo = W.normal_bf16(rng, p["permuted"].shape)
    probs = rng.standard_normal((T, K)).astype(np.float32)
    ori = W.normal_bf16(rng, (T, H))
    shared = W.normal_bf16(rng, (T, H))
    cv = W.uniform_bf16(rng, (Nc, H), -1, 1)
    # per-token coefficients
    a1 = rng.random(T).astype(np.float32)
    a2 = rng.random(T).astype(np.float32)
    got, ref, ref64 = _combine_both(moe_lib, eo, p["row_of_slot"], ids, probs, E, Z=Z, C=C, Nc=Nc,
                                    ori=ori, a1=a1, a2=a2, strides=(1, 0, 0), cv=cv,
                                    shared=shared)
    assert_rel(f64(got), ref64, 1e-2, "special per-token")
    # the page's (const_num, H) coefficient layout
    b1 = rng.uniform(-1, 1, (Nc, H)).astype(np.float32)
    b2 = rng.uniform(-1, 1, (Nc, H)).astype(np.float32)
    got, ref, ref64 = _combine_both(moe_lib, eo, p["row_of_slot"], ids, probs, E, Z=Z, C=C, Nc=Nc,
                                    ori=ori, a1=b1, a2=b2, strides=(0, H, 1), cv=cv)
    assert_rel(f64(got), ref64, 1e-2, "special per-(c,h)")


def test_combine_closed_forms(moe_lib):
    rng = np.random.default_rng(22)
    T, K, E, H, Z, C = 256, 4, 8, 64, 2, 2
    shared = W.normal_bf16(rng, (T, H))
    eo = W.normal_bf16(rng, (T * K, H))
    zero_ids = rng.integers(E, E + Z, size=(T, K)).astype(np.int32)
    ros = np.full((T, K), -1, np.int32)
    got, _, _ = _combine_both(moe_lib, eo, ros, zero_ids, rng.standard_normal((T, K)).astype(np.float32),
                              E, Z=Z, C=C, ori=W.normal_bf16(rng, (T, H)), shared=shared)
    np.testing.assert_array_equal(got, shared)   # zero experts leave the shared row only


def test_combine_config4_with_row_map(moe_lib):
    g = W.gen_c4()
    c = g["cfg"]
    R, El, H = c["R"], c["E_local"], c["H"]
    # GPU: reorder, then combine the expert-major buffer through inv_perm
    r = moe_lib.reorder_alloc(to_dev_bf16(g["x_rank_major"]), to_dev(g["counts"]), R, El)
    sp, keep = _special(moe_lib, c["num_zero"], c["num_copy"], c["num_const"], g["ori_x"],
                        g["alpha1"], g["alpha2"], (1, 0, 0), g["const_v"])
    out = moe_lib.combine_alloc(r["y"], to_dev(g["slot_src_row"]), to_dev(g["expert_ids"]),
                                to_dev(g["probs"]), El, row_map=r["inv_perm"], special=sp,
                                shared_x=to_dev_bf16(g["shared_x"]))
    torch.cuda.synchronize()
    ro = oracle.reorder(g["x_rank_major"], g["counts"], R, El)
    ref, ref64 = oracle.combine(ro["y"], g["slot_src_row"], g["expert_ids"], g["probs"], El,
                                row_map=ro["inv_perm"], num_zero=c["num_zero"],
                                num_copy=c["num_copy"], num_const=c["num_const"], ori_x=g["ori_x"],
                                alpha1=g["alpha1"], alpha2=g["alpha2"], alpha_strides=(1, 0, 0),
                                const_v=g["const_v"], shared_x=g["shared_x"])
    got = bits(out)
    # shared term and signed special terms cancel: near-zero outputs differ by many
    # ulps, so only the relative bound applies here
    assert_rel(f64(got), ref64, 1e-2, "config 4 combine")
