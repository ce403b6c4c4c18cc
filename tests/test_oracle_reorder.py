"""Pins of the oracle's rank-major -> expert-major reorder: hand-worked
fixtures, numpy's stable lexsort by (expert, rank) (a library stable sort),
the identity special cases and the agreement of the page's two formulations."""
import json
import os

import numpy as np
import pytest

import moe_workloads as W
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _lexsort_reference(counts, R, El):
    """Expert-major order = stable sort of the rank-major rows by (expert, rank)."""
    r_lab = np.repeat(np.repeat(np.arange(R), El), counts)
    e_lab = np.repeat(np.tile(np.arange(El), R), counts)
    return np.lexsort((r_lab, e_lab))  # last key is primary; stable


def test_hand_worked_fixtures():
    g = json.load(open(os.path.join(GOLD, "reorder_tiny.json")))
    for sfx in ("", "_b"):
        cnt = np.array(g["counts" + sfx], np.int32)
        r = oracle.reorder(None, cnt, g["R"], g["E_local"], rows=False)
        np.testing.assert_array_equal(r["perm"], g["perm" + sfx])
        np.testing.assert_array_equal(r["tokens_per_expert"], g["tokens_per_expert" + sfx])


@pytest.mark.parametrize("R,El,N,seed", [(1, 1, 10, 0), (1, 7, 100, 1), (5, 1, 77, 2),
                                         (8, 32, 4000, 3), (3, 5, 0, 4), (16, 8, 999, 5)])
def test_against_lexsort_and_vectorized(R, El, N, seed):
    cnt = W.make_rank_major_counts(R, El, N, seed)
    x = W.normal_bf16(np.random.default_rng(seed), (N, 16))
    r = oracle.reorder(x, cnt, R, El)
    ref = _lexsort_reference(cnt, R, El)
    np.testing.assert_array_equal(r["perm"], ref)
    v = oracle.reorder_index_vectorized(cnt, R, El)
    np.testing.assert_array_equal(v["perm"], r["perm"])
    np.testing.assert_array_equal(v["tokens_per_expert"], cnt.reshape(R, El).sum(0))
    np.testing.assert_array_equal(r["tokens_per_expert"], cnt.reshape(R, El).sum(0))
    np.testing.assert_array_equal(r["expert_offsets"],
                                  np.concatenate([[0], np.cumsum(cnt.reshape(R, El).sum(0))]))
    np.testing.assert_array_equal(r["inv_perm"][r["perm"]], np.arange(N))
    np.testing.assert_array_equal(r["y"], x[ref])
    if R == 1 or El == 1:
        np.testing.assert_array_equal(r["perm"], np.arange(N))


def test_capacity_past_total():
    cnt = np.array([2, 0, 1, 3], np.int32)
    x = np.arange(9 * 4, dtype=np.uint16).reshape(9, 4)
    r = oracle.reorder(x, cnt, 2, 2, N=9)
    assert np.all(r["perm"][6:] == -1) and np.all(r["inv_perm"][6:] == -1)
    assert np.all(r["y"][6:] == 0)


def test_config4_counts():
    c = W.gen_c4(with_rows=False)
    cfg = c["cfg"]
    r = oracle.reorder(None, c["counts"], cfg["R"], cfg["E_local"], rows=False)
    np.testing.assert_array_equal(r["perm"], _lexsort_reference(c["counts"], cfg["R"], cfg["E_local"]))
    assert int(c["counts"].sum()) == cfg["N"]
