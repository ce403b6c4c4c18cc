"""Pins of the oracle's x_active_mask reading (the combine_v2 page, 参数说明: a
[BS] mask with its trues first marks the tokens that take part, a [BS, K]
mask the slots; a token whose K flags are all false takes no part): a prefix
mask gives exactly the permute / combine of the active prefix, an all-true
mask changes nothing, an all-false [T, K] row leaves only the shared row, a
[T] mask equals the [T, K] mask that repeats it, and the masked combine
backward is the derivative of the masked combine."""
import numpy as np
import pytest

import moe_workloads as W
import oracle


def _data(seed, T=40, K=4, E=9, H=24):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    return rng, ids, W.normal_bf16(rng, (T, H)), rng.standard_normal((T, K)).astype(np.float32)


@pytest.mark.parametrize("n_active", [0, 1, 17, 40])
def test_prefix_mask_is_the_permute_of_the_prefix(n_active):
    rng, ids, x, _ = _data(1)
    T, K = ids.shape
    mask = np.arange(T) < n_active
    full = oracle.permute(x, ids, 9, active_mask=mask)
    pre = oracle.permute(x[:n_active], ids[:n_active], 9)
    n = int(pre["expert_offsets"][-1])
    np.testing.assert_array_equal(full["expert_counts"], pre["expert_counts"])
    np.testing.assert_array_equal(full["expert_offsets"], pre["expert_offsets"])
    np.testing.assert_array_equal(full["row_of_slot"][:n_active], pre["row_of_slot"])
    assert np.all(full["row_of_slot"][n_active:] == -1)
    np.testing.assert_array_equal(full["sorted_slot"][:n], pre["sorted_slot"][:n])
    assert np.all(full["sorted_slot"][n:] == -1)
    np.testing.assert_array_equal(full["permuted"][:n], pre["permuted"][:n])


def test_prefix_mask_is_the_combine_of_the_prefix_plus_shared_rows():
    rng, ids, x, probs = _data(2)
    T, K = ids.shape
    n_active = 23
    mask = np.arange(T) < n_active
    p = oracle.permute(x, ids, 9, active_mask=mask)
    shared = W.normal_bf16(rng, x.shape)
    out, out64 = oracle.combine(p["permuted"], p["row_of_slot"], ids, probs, 9, shared_x=shared,
                                active_mask=mask)
    pp = oracle.permute(x[:n_active], ids[:n_active], 9)
    o2, o264 = oracle.combine(pp["permuted"], pp["row_of_slot"], ids[:n_active], probs[:n_active],
                              9, shared_x=shared[:n_active])
    np.testing.assert_array_equal(out[:n_active], o2)
    np.testing.assert_array_equal(out[n_active:], shared[n_active:])


def test_all_true_changes_nothing_and_token_mask_repeats():
    rng, ids, x, probs = _data(3)
    T, K = ids.shape
    p0 = oracle.permute(x, ids, 9)
    p1 = oracle.permute(x, ids, 9, active_mask=np.ones(T, bool))
    p2 = oracle.permute(x, ids, 9, active_mask=np.ones((T, K), bool))
    for key in p0:
        np.testing.assert_array_equal(p0[key], p1[key])
        np.testing.assert_array_equal(p0[key], p2[key])
    tok = rng.random(T) < 0.6
    a = oracle.permute(x, ids, 9, active_mask=tok)
    b = oracle.permute(x, ids, 9, active_mask=np.repeat(tok[:, None], K, 1))
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_slot_mask_and_all_false_rows():
    """[T, K]: a masked slot adds nothing (zero, copy and const slots too); a
    token with all K flags false keeps only its shared row."""
    rng, ids, x, probs = _data(4, T=30, K=3, E=6, H=16)
    T, K = ids.shape
    E, Z, C, NC = 6, 1, 1, 1
    ids[::4, 0] = E + rng.integers(0, Z + C + NC, size=ids[::4, 0].shape)
    ori = W.normal_bf16(rng, x.shape)
    cv = W.normal_bf16(rng, (NC, x.shape[1]))
    a1 = rng.random(T).astype(np.float32)
    a2 = rng.random(T).astype(np.float32)
    shared = W.normal_bf16(rng, x.shape)
    m = rng.random((T, K)) < 0.7
    m[5] = False
    p = oracle.permute(x, ids, E, active_mask=m)
    kw = dict(num_zero=Z, num_copy=C, num_const=NC, ori_x=ori, alpha1=a1, alpha2=a2,
              alpha_strides=(1, 0, 0), const_v=cv, shared_x=shared)
    out, out64 = oracle.combine(p["permuted"], p["row_of_slot"], ids, probs, E, active_mask=m, **kw)
    np.testing.assert_array_equal(out[5], shared[5])
    # the same sum with the masked slots' weights set to zero
    pz = np.where(m, probs, np.float32(0))
    q = oracle.permute(x, ids, E)
    _, ref64 = oracle.combine(q["permuted"], q["row_of_slot"], ids, pz, E, **kw)
    np.testing.assert_allclose(out64, ref64, rtol=0, atol=1e-12)


def test_masked_combine_grad_is_the_derivative_of_the_masked_combine():
    rng, ids, x, _ = _data(5, T=20, K=3, E=7, H=16)
    T, K = ids.shape
    probs = (rng.integers(-1024, 1025, size=(T, K)) / 1024.0).astype(np.float32)  # p +- 1 exact
    m = rng.random((T, K)) < 0.6
    p = oracle.permute(x, ids, 7, active_mask=m)
    eo = W.normal_bf16(rng, p["permuted"].shape)
    g = W.normal_bf16(rng, x.shape)
    r = oracle.combine_grad(g, eo, p["row_of_slot"], ids, probs, 7, active_mask=m)
    gf = W.f32_from_bf16(g).astype(np.float64)
    for t in range(T):
        for k in range(K):
            hi, lo = probs.copy(), probs.copy()
            hi[t, k] += 1.0
            lo[t, k] -= 1.0
            _, a = oracle.combine(eo, p["row_of_slot"], ids, hi, 7, active_mask=m)
            _, b = oracle.combine(eo, p["row_of_slot"], ids, lo, 7, active_mask=m)
            fd = (np.sum(a * gf) - np.sum(b * gf)) / 2.0
            assert abs(fd - r["d_probs"][t, k]) <= 1e-9 * (1 + abs(fd))
            if not m[t, k]:
                assert r["d_probs"][t, k] == 0.0
