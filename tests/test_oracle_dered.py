"""Pins of the oracle's deredundency index math and whiteboard scatter-add
(coverage page of hyper_parallel expert_parallel.py:
_generate_deredundency_dispatch_indices, _scale_by_router_coeff,
_scatter_add_first_dim): hand-worked fixtures, the block loop against the
page's vectorised form, invariants of the selection, the single-source closed
form, agreement with the (independently pinned) rank-major reorder when one
destination takes every expert, and numpy's add.at for the scatter-add."""
import json
import os

import numpy as np
import pytest

import moe_workloads as W
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "dered_tiny.json")


def test_hand_worked_fixtures():
    for case in json.load(open(GOLD))["cases"]:
        c = np.array(case["counts"], np.int32)
        for form in ("loop", "vectorized"):
            idx, cbd, tot = oracle.dered_indices(c, case["expert_start"], case["iep_size"],
                                                 case["num_local"], form=form)
            assert tot == len(case["indices"])
            np.testing.assert_array_equal(idx[:tot], case["indices"])
            assert np.all(idx[tot:] == -1)
            np.testing.assert_array_equal(cbd, case["counts_by_dest"])


def _random(seed, oep, E, zero_frac=0.3, hi=40):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, hi, size=(oep, E)).astype(np.int32)
    c[rng.random((oep, E)) < zero_frac] = 0
    return rng, c


@pytest.mark.parametrize("oep,E,iep,El,start,seed", [
    (1, 8, 2, 4, 0, 0), (4, 64, 4, 8, 16, 1), (8, 256, 8, 4, 128, 2), (3, 10, 1, 1, 9, 3),
    (16, 32, 2, 16, 0, 4),
])
def test_loop_equals_the_vectorised_form_and_invariants(oep, E, iep, El, start, seed):
    rng, c = _random(seed, oep, E)
    c[0, start] = -3                                          # negative counts read as 0
    a = oracle.dered_indices(c, start, iep, El)
    b = oracle.dered_indices(c, start, iep, El, form="vectorized")
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    assert a[2] == b[2]
    idx, cbd, tot = a
    cc = np.maximum(c, 0)
    sel = cc[:, start:start + iep * El]
    np.testing.assert_array_equal(cbd, sel.sum(0))
    assert tot == int(sel.sum())
    got = idx[:tot]
    assert len(np.unique(got)) == tot                         # distinct rows
    # every selected gathered row maps back to (source, expert) in the range, and
    # the order is (destination, local expert, source, row)
    flat = np.concatenate([[0], np.cumsum(cc.reshape(-1))])
    cell = np.searchsorted(flat, got, side="right") - 1
    s_of, e_of = cell // E, cell % E
    assert np.all((e_of >= start) & (e_of < start + iep * El))
    key = np.stack([e_of - start, s_of, got], 1)              # (d*El + l, s, row)
    assert np.all(np.diff(key[:, 0]) >= 0)
    order = np.lexsort((key[:, 2], key[:, 1], key[:, 0]))
    np.testing.assert_array_equal(order, np.arange(tot))


def test_single_source_full_range_is_the_identity():
    _, c = _random(5, 1, 48)
    idx, cbd, tot = oracle.dered_indices(c, 0, 6, 8)
    np.testing.assert_array_equal(idx, np.arange(tot))
    np.testing.assert_array_equal(cbd, c[0])


@pytest.mark.parametrize("R,El,seed", [(8, 32, 6), (3, 5, 7)])
def test_one_destination_every_expert_is_the_reorder(R, El, seed):
    """With iep_size = 1 and the whole expert range, the gathered buffer is a
    rank-major receive buffer and the selection is its expert-major order."""
    _, c = _random(seed, R, El)
    idx, cbd, tot = oracle.dered_indices(c, 0, 1, El)
    ro = oracle.reorder(None, c.reshape(-1), R, El, rows=False)
    np.testing.assert_array_equal(idx[:tot], ro["perm"][:tot])
    np.testing.assert_array_equal(cbd, ro["tokens_per_expert"])


def test_empty_selection():
    c = np.zeros((3, 8), np.int32)
    c[:, :4] = 5
    idx, cbd, tot = oracle.dered_indices(c, 4, 2, 2, capacity=6)
    assert tot == 0 and np.all(idx == -1) and not cbd.any()


def test_scatter_add_against_numpy_add_at():
    rng = np.random.default_rng(8)
    n, H, G = 300, 24, 120
    src = W.normal_bf16(rng, (n, H))
    ix = rng.integers(-2, G + 2, size=n).astype(np.int32)     # duplicates and out-of-range
    coeff = rng.standard_normal(n).astype(np.float32)
    out, out64 = oracle.scatter_add_rows(src, ix, G, coeff)
    ref = np.zeros((G, H))
    ok = (ix >= 0) & (ix < G)
    np.add.at(ref, ix[ok], coeff[ok, None].astype(np.float64) * W.f32_from_bf16(src[ok]))
    np.testing.assert_allclose(out64, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(out, oracle.f64_to_bf16(ref))


def test_scatter_of_distinct_rows_and_adjoint():
    rng = np.random.default_rng(9)
    c = rng.integers(0, 30, size=(4, 16)).astype(np.int32)
    idx, _, tot = oracle.dered_indices(c, 4, 2, 4)
    G = int(c.sum())
    H = 32
    src = W.normal_bf16(rng, (tot, H))
    # no coefficient: the selected rows come back unchanged, every other row is 0
    out, _ = oracle.scatter_add_rows(src, idx[:tot], G)
    np.testing.assert_array_equal(out[idx[:tot]], src)
    rest = np.setdiff1d(np.arange(G), idx[:tot])
    assert not out[rest].any()
    coeff = rng.standard_normal(tot).astype(np.float32)
    _, o64 = oracle.scatter_add_rows(src, idx[:tot], G, coeff)
    gm = rng.standard_normal((G, H))
    lhs = float(np.sum(o64 * gm))
    rhs = float(np.sum(coeff[:, None].astype(np.float64) * W.f32_from_bf16(src) * gm[idx[:tot]]))
    assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs))
