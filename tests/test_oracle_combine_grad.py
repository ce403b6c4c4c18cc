"""Pins of the oracle's combine backward with special and shared experts: the
derivative of the oracle combine's fp64 output (central differences, exact
because the combine is linear in each input on its own), the whole-tensor
adjoint identities that linearity gives, the alpha layouts as sums of one
expanded per-(t, c, h) layout, agreement with the unpermute backward when no
special expert is used, the row map, and closed forms for copy / zero slots."""
import numpy as np
import pytest

import moe_workloads as W
import oracle

Z, C, NC = 2, 2, 3           # zero, copy and const experts
LAYOUTS = {                  # alpha element (t, c, h) at t*st + c*sc + h*sh
    "per_token": lambda T, H: ((1, 0, 0), T),
    "const_by_h": lambda T, H: ((0, H, 1), NC * H),
    "token_by_const": lambda T, H: ((NC, 1, 0), T * NC),
    "scalar": lambda T, H: ((0, 0, 0), 1),
}


def _grid(rng, shape):
    """fp32 values on a 2^-10 grid in [-1, 1]: adding +-1 stays exact."""
    return (rng.integers(-1024, 1025, size=shape) / 1024.0).astype(np.float32)


def _setup(seed, layout="per_token", T=14, K=4, E=5, H=24):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, E + Z + C + NC + 1, size=(T, K)).astype(np.int32)
    ids[0, :4] = [0, E, E + Z, E + Z + C]            # one of each kind in token 0
    strides, n_alpha = LAYOUTS[layout](T, H)
    p = oracle.permute(None, ids, E, rows=False)
    N = int(p["expert_offsets"][-1])
    return dict(
        ids=ids, E=E, ros=p["row_of_slot"], probs=_grid(rng, (T, K)),
        eo=W.normal_bf16(rng, (max(N, 1), H)), g=W.normal_bf16(rng, (T, H)),
        ori=W.normal_bf16(rng, (T, H)), cv=W.normal_bf16(rng, (NC, H)),
        a1=_grid(rng, n_alpha), a2=_grid(rng, n_alpha), shared=W.normal_bf16(rng, (T, H)),
        strides=strides)


def _loss(d, **over):
    """L = sum(out_f64 * g): the scalar whose gradient the backward returns."""
    a = dict(d, **over)
    _, out64 = oracle.combine(a["eo"], a["ros"], a["ids"], a["probs"], a["E"], num_zero=Z,
                              num_copy=C, num_const=NC, ori_x=a["ori"], alpha1=a["a1"],
                              alpha2=a["a2"], alpha_strides=a["strides"], const_v=a["cv"],
                              shared_x=a["shared"], row_map=a.get("row_map"))
    return float(np.sum(out64 * W.f32_from_bf16(d["g"]).astype(np.float64)))


def _grad(d):
    return oracle.combine_grad(d["g"], d["eo"], d["ros"], d["ids"], d["probs"], d["E"],
                               num_zero=Z, num_copy=C, num_const=NC, ori_x=d["ori"],
                               alpha1=d["a1"], alpha2=d["a2"], alpha_strides=d["strides"],
                               const_v=d["cv"], row_map=d.get("row_map"))


PLUS, MINUS = np.uint16(0x3F80), np.uint16(0xBF80)     # bf16 +1 and -1


def _fd_bf16(d, key, idx):
    """Central difference in one bf16 element, taken between -1 and +1."""
    hi, lo = d[key].copy(), d[key].copy()
    hi[idx], lo[idx] = PLUS, MINUS
    return (_loss(d, **{key: hi}) - _loss(d, **{key: lo})) / 2.0


def _fd_f32(d, key, idx):
    hi, lo = d[key].copy(), d[key].copy()
    hi[idx] += 1.0
    lo[idx] -= 1.0
    return (_loss(d, **{key: hi}) - _loss(d, **{key: lo})) / 2.0


def _close(a, b):
    assert abs(a - b) <= 1e-10 * (1 + abs(a) + abs(b)), (a, b)


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_gradients_are_the_finite_differences_of_the_combine(layout):
    d = _setup(1, layout)
    r = _grad(d)
    T, K = d["ids"].shape
    H = d["g"].shape[1]
    rng = np.random.default_rng(2)
    for t in range(T):
        for k in range(K):
            _close(_fd_f32(d, "probs", (t, k)), r["d_probs"][t, k])
    for _ in range(12):
        t, h = int(rng.integers(T)), int(rng.integers(H))
        _close(_fd_bf16(d, "ori", (t, h)), r["d_ori_x"][t, h])
        _close(_fd_bf16(d, "shared", (t, h)), r["d_shared"][t, h])
        c = int(rng.integers(NC))
        _close(_fd_bf16(d, "cv", (c, h)), r["d_const_v"][c, h])
        i = int(rng.integers(d["a1"].size))
        _close(_fd_f32(d, "a1", i), r["d_alpha1"][i])
        _close(_fd_f32(d, "a2", i), r["d_alpha2"][i])
    rows = np.flatnonzero(r["row_written"])
    assert rows.size > 0
    for row in rows[:: max(1, rows.size // 10)]:
        h = int(rng.integers(H))
        _close(_fd_bf16(d, "eo", (row, h)), r["d_expert_out"][row, h])
    # rows no slot references: the combine does not depend on them
    assert not np.any(r["d_expert_out"][~r["row_written"]])


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_adjoint_identities(layout):
    """The combine is linear in each input alone, so L(x) - L(x = 0) = <dL/dx, x>."""
    d = _setup(3, layout, T=20, K=6, H=32)
    r = _grad(d)
    f = lambda b: W.f32_from_bf16(b).astype(np.float64)
    L = _loss(d)
    zero = lambda key: np.zeros_like(d[key])
    pairs = [("eo", f(d["eo"]), r["d_expert_out"]), ("ori", f(d["ori"]), r["d_ori_x"]),
             ("cv", f(d["cv"]), r["d_const_v"]), ("shared", f(d["shared"]), r["d_shared"]),
             ("a1", d["a1"].astype(np.float64), r["d_alpha1"]),
             ("a2", d["a2"].astype(np.float64), r["d_alpha2"]),
             ("probs", d["probs"].astype(np.float64), r["d_probs"])]
    for key, x, dx in pairs:
        _close(L - _loss(d, **{key: zero(key)}), float(np.sum(x * dx)))


@pytest.mark.parametrize("layout", ["per_token", "const_by_h", "token_by_const", "scalar"])
def test_alpha_layouts_sum_the_expanded_gradient(layout):
    """Any alpha layout is a broadcast of one element per (t, c, h); its
    gradient is the sum of the expanded layout's gradient over the elements
    that share a storage location."""
    d = _setup(5, layout, T=10, K=5, H=16)
    T, H = d["g"].shape
    st, sc, sh = d["strides"]
    tt, cc, hh = np.meshgrid(np.arange(T), np.arange(NC), np.arange(H), indexing="ij")
    where = tt * st + cc * sc + hh * sh                         # [T, NC, H] storage index
    ex = dict(d, a1=d["a1"][where].reshape(-1), a2=d["a2"][where].reshape(-1),
              strides=(NC * H, H, 1))
    _close(_loss(d), _loss(ex))
    r, rx = _grad(d), _grad(ex)
    for key in ("d_alpha1", "d_alpha2"):
        want = np.zeros(d["a1"].size)
        np.add.at(want, where.reshape(-1), rx[key])
        np.testing.assert_allclose(r[key], want, rtol=1e-12, atol=1e-12)
    for key in ("d_probs", "d_ori_x", "d_const_v"):
        np.testing.assert_allclose(r[key], rx[key], rtol=1e-12, atol=1e-12)


def test_without_special_experts_equals_the_unpermute_backward():
    rng = np.random.default_rng(7)
    T, K, E, H = 30, 4, 9, 40
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    ids[3, 1] = -1
    p = oracle.permute(None, ids, E, rows=False)
    N = int(p["expert_offsets"][-1])
    eo, g = W.normal_bf16(rng, (N, H)), W.normal_bf16(rng, (T, H))
    probs = rng.standard_normal((T, K)).astype(np.float32)
    r = oracle.combine_grad(g, eo, p["row_of_slot"], ids, probs, E)
    dperm, dprobs, dperm64, dprobs64 = oracle.unpermute_grad(g, eo, p["row_of_slot"], probs)
    np.testing.assert_array_equal(r["d_expert_out"], dperm64)
    np.testing.assert_array_equal(r["d_probs"], dprobs64)
    assert r["row_written"].all()
    assert not r["d_ori_x"].any() and r["d_const_v"].size == 0


def test_row_map_moves_the_expert_gradient_with_the_row():
    """Reading expert rows through a row map equals reading a buffer whose rows
    were moved by that map; the expert gradient moves with them."""
    rng = np.random.default_rng(8)
    T, K, E, H = 25, 3, 6, 16
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    p = oracle.permute(None, ids, E, rows=False)
    N = int(p["expert_offsets"][-1])
    eo, g = W.normal_bf16(rng, (N, H)), W.normal_bf16(rng, (T, H))
    probs = rng.random((T, K)).astype(np.float32)
    rmap = rng.permutation(N).astype(np.int32)
    moved = np.empty_like(eo)
    moved[rmap] = eo
    direct = oracle.combine_grad(g, eo, p["row_of_slot"], ids, probs, E)
    mapped = oracle.combine_grad(g, moved, p["row_of_slot"], ids, probs, E, row_map=rmap)
    np.testing.assert_array_equal(mapped["d_expert_out"][rmap], direct["d_expert_out"])
    np.testing.assert_array_equal(mapped["d_probs"], direct["d_probs"])


def test_copy_and_zero_closed_forms():
    """All slots copy experts: d_ori_x = (sum_k p) g and d_probs = <g, ori_x>;
    all slots zero experts: every derivative but d_shared is 0."""
    rng = np.random.default_rng(9)
    T, K, E, H = 12, 3, 4, 20
    g, ori = W.normal_bf16(rng, (T, H)), W.normal_bf16(rng, (T, H))
    gf, of = W.f32_from_bf16(g).astype(np.float64), W.f32_from_bf16(ori).astype(np.float64)
    probs = _grid(rng, (T, K))
    ids = (E + Z + rng.integers(0, C, size=(T, K))).astype(np.int32)
    ros = np.full((T, K), -1, np.int32)
    r = oracle.combine_grad(g, None, ros, ids, probs, E, num_zero=Z, num_copy=C, ori_x=ori)
    np.testing.assert_allclose(r["d_ori_x"], probs.astype(np.float64).sum(1)[:, None] * gf,
                               rtol=1e-14, atol=0)
    np.testing.assert_allclose(r["d_probs"], np.repeat(np.sum(gf * of, 1)[:, None], K, 1),
                               rtol=1e-14, atol=0)
    zids = (E + rng.integers(0, Z, size=(T, K))).astype(np.int32)
    r = oracle.combine_grad(g, None, ros, zids, probs, E, num_zero=Z, num_copy=C, ori_x=ori)
    assert not r["d_probs"].any() and not r["d_ori_x"].any()
    np.testing.assert_array_equal(r["d_shared"], gf)


def test_bad_alpha_extent_is_rejected():
    d = _setup(4, "const_by_h")
    with pytest.raises(Exception):
        oracle.combine_grad(d["g"], d["eo"], d["ros"], d["ids"], d["probs"], d["E"],
                            num_zero=Z, num_copy=C, num_const=NC, ori_x=d["ori"],
                            alpha1=d["a1"][:-1], alpha2=d["a2"][:-1],
                            alpha_strides=d["strides"], const_v=d["cv"])
