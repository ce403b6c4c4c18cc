"""GPU parity of moe_unpermute_combine_grad (the combine's backward with zero,
copy and const experts) against the oracle: expert-row gradients bit-exact
(correctly rounded products on both sides), every other output within the
1e-2 relative bound (fp32 accumulation against fp64)."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_rel, bits, f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

LAYOUTS = {   # alpha element (t, c, h) at t*st + c*sc + h*sh, and its element count
    "per_token": lambda T, H, nc: ((1, 0, 0), T),
    "const_by_h": lambda T, H, nc: ((0, H, 1), nc * H),
    "token_by_const": lambda T, H, nc: ((nc, 1, 0), T * nc),
    "per_const": lambda T, H, nc: ((0, 1, 0), nc),
    "scalar": lambda T, H, nc: ((0, 0, 0), 1),
    "const_by_h_padded": lambda T, H, nc: ((0, H + 8, 1), nc * (H + 8)),
}


def _case(seed, T, K, E, H, Z, C, NC, layout, drop=0.05, special=0.3):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    m = rng.random((T, K)) < special
    ids[m] = E + rng.integers(0, Z + C + NC, size=int(m.sum()))
    ids[rng.random((T, K)) < drop] = -1
    strides, n_alpha = LAYOUTS[layout](T, H, NC)
    p = oracle.permute(None, ids, E, rows=False)
    N = int(p["expert_offsets"][-1])
    return dict(ids=ids, E=E, Z=Z, C=C, NC=NC, ros=p["row_of_slot"], N=N,
                probs=rng.standard_normal((T, K)).astype(np.float32),
                eo=W.normal_bf16(rng, (N, H)), g=W.normal_bf16(rng, (T, H)),
                ori=W.normal_bf16(rng, (T, H)), cv=W.normal_bf16(rng, (NC, H)),
                a1=rng.uniform(-1, 1, n_alpha).astype(np.float32),
                a2=rng.uniform(-1, 1, n_alpha).astype(np.float32), strides=strides)


def _run(moe, d, row_map=None, want=("d_expert_out", "d_probs", "d_ori_x", "d_alpha",
                                     "d_const_v")):
    T, K = d["ids"].shape
    H = d["g"].shape[1]
    print(f"combine_grad T={T} K={K} E={d['E']} H={H} special={d['Z']},{d['C']},{d['NC']} "
          f"strides={d['strides']} row_map={row_map is not None}", flush=True)
    nsp = d["Z"] + d["C"] + d["NC"]
    keep = [to_dev_bf16(d["ori"]), to_dev(d["a1"]), to_dev(d["a2"]), to_dev_bf16(d["cv"])]
    sp = moe.make_special(d["Z"], d["C"], d["NC"], keep[0], keep[1], keep[2], d["strides"],
                          keep[3]) if nsp else None
    sentinel = torch.full((d["N"], H), 0x1234, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    got = moe.combine_grad_alloc(to_dev_bf16(d["g"]), to_dev_bf16(d["eo"]), to_dev(d["ros"]),
                                 to_dev(d["ids"]), to_dev(d["probs"]), d["E"],
                                 row_map=to_dev(row_map) if row_map is not None else None,
                                 special=sp, alpha_numel=d["a1"].size, d_expert_out=sentinel,
                                 want=want)
    torch.cuda.synchronize()
    ref = oracle.combine_grad(d["g"], d["eo"], d["ros"], d["ids"], d["probs"], d["E"],
                              row_map=row_map, num_zero=d["Z"], num_copy=d["C"],
                              num_const=d["NC"], ori_x=d["ori"], alpha1=d["a1"],
                              alpha2=d["a2"], alpha_strides=d["strides"], const_v=d["cv"])
    assert_rel(got["d_probs"].cpu().numpy(), ref["d_probs"], 1e-2, "d_probs")
    if "d_expert_out" in got:
        deo = bits(got["d_expert_out"])
        w = ref["row_written"]
        np.testing.assert_array_equal(deo[w], oracle.f64_to_bf16(ref["d_expert_out"][w]))
        assert np.all(deo[~w] == 0x1234), "rows no slot references must stay untouched"
    if "d_ori_x" in got:
        assert_rel(f64(bits(got["d_ori_x"])), ref["d_ori_x"], 1e-2, "d_ori_x")
    if "d_const_v" in got:
        assert_rel(f64(bits(got["d_const_v"])), ref["d_const_v"], 1e-2, "d_const_v")
    if "d_alpha1" in got:
        st, sc, sh = d["strides"]
        tt, cc, hh = np.meshgrid(np.arange(T), np.arange(d["NC"]), np.arange(H), indexing="ij")
        used = np.unique((tt * st + cc * sc + hh * sh).reshape(-1))   # elements alpha reads
        for key in ("d_alpha1", "d_alpha2"):
            assert_rel(got[key].cpu().numpy()[used], ref[key][used], 1e-2, key)
    return got, ref


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_combine_grad_layouts(moe_lib, layout):
    _run(moe_lib, _case(1, T=300, K=6, E=8, H=136, Z=2, C=2, NC=3, layout=layout))


@pytest.mark.parametrize("T,K,E,H,NC,seed", [
    (1, 1, 1, 8, 1, 2),            # one token, one slot
    (2000, 8, 32, 1160, 9, 3),     # several hidden tiles with a ragged tail, 3 const groups
    (777, 16, 40, 520, 5, 4),      # K = 16, many segments
    (901, 8, 24, 2120, 3, 6),      # 4 waves per token, 265 chunks: uneven parts
])
def test_combine_grad_shapes(moe_lib, T, K, E, H, NC, seed):
    for layout in ("per_token", "const_by_h"):
        _run(moe_lib, _case(seed, T=T, K=K, E=E, H=H, Z=1, C=2, NC=NC, layout=layout))


def test_combine_grad_row_map(moe_lib):
    d = _case(5, T=400, K=4, E=12, H=264, Z=2, C=1, NC=2, layout="per_token")
    rng = np.random.default_rng(6)
    rmap = rng.permutation(d["N"]).astype(np.int32)
    moved = np.empty_like(d["eo"])
    moved[rmap] = d["eo"]
    d["eo"] = moved
    _run(moe_lib, d, row_map=rmap)


def test_combine_grad_without_special_matches_unpermute_grad(moe_lib):
    d = _case(7, T=500, K=6, E=16, H=256, Z=0, C=0, NC=0, layout="per_token", special=0.0)
    got, _ = _run(moe_lib, d, want=("d_expert_out", "d_probs"))
    dp, dpr = moe_lib.unpermute_grad_alloc(to_dev_bf16(d["g"]), to_dev_bf16(d["eo"]),
                                           to_dev(d["ros"]), to_dev(d["probs"]))
    torch.cuda.synchronize()
    w = oracle.combine_grad(d["g"], d["eo"], d["ros"], d["ids"], d["probs"], d["E"])["row_written"]
    np.testing.assert_array_equal(bits(got["d_expert_out"])[w], bits(dp)[w])


def test_combine_grad_partial_outputs_and_empty(moe_lib):
    d = _case(8, T=120, K=4, E=6, H=64, Z=1, C=1, NC=2, layout="const_by_h")
    _run(moe_lib, d, want=("d_probs", "d_const_v"))
    _run(moe_lib, d, want=("d_probs", "d_alpha"))
    _run(moe_lib, d, want=("d_probs",))
    # only special slots: nothing routed to a real expert
    e = _case(9, T=50, K=3, E=4, H=32, Z=1, C=1, NC=1, layout="per_token", special=1.0, drop=0.0)
    assert e["N"] == 0
    _run(moe_lib, e)


def test_combine_grad_unsupported_alpha_layout(moe_lib):
    """[T, H] alpha (strides (H, 0, 1)): its d_alpha has no kernel and is refused;
    the other gradients are still available for it."""
    T, H = 64, 32
    d = _case(10, T=T, K=3, E=5, H=H, Z=1, C=1, NC=1, layout="per_token")
    rng = np.random.default_rng(11)
    d["a1"] = rng.uniform(-1, 1, T * H).astype(np.float32)
    d["a2"] = rng.uniform(-1, 1, T * H).astype(np.float32)
    d["strides"] = (H, 0, 1)
    with pytest.raises(moe_lib.MoeError) as e:
        _run(moe_lib, d)
    assert e.value.status == 2
    _run(moe_lib, d, want=("d_expert_out", "d_probs", "d_ori_x", "d_const_v"))


def test_combine_grad_receive_buffer_workload(moe_lib):
    """The receive-buffer workload (T=4608, K=8, H=4096, 4 zero / 4 copy / 4 const
    experts, per-token alpha), read through the reorder's inverse map."""
    g = W.gen_c4()
    c = g["cfg"]
    R, El, H, T = c["R"], c["E_local"], c["H"], c["T"]
    ro = oracle.reorder(g["x_rank_major"], g["counts"], R, El)
    rng = np.random.default_rng(12)
    d = dict(ids=g["expert_ids"], E=El, Z=c["num_zero"], C=c["num_copy"], NC=c["num_const"],
             ros=g["slot_src_row"], N=c["N"], probs=g["probs"], eo=ro["y"],
             g=W.normal_bf16(rng, (T, H)), ori=g["ori_x"], cv=g["const_v"], a1=g["alpha1"],
             a2=g["alpha2"], strides=(1, 0, 0))
    _run(moe_lib, d, row_map=ro["inv_perm"])
