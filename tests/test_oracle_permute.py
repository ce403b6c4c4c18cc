"""Pins of the oracle's token permute: a hand-worked fixture, numpy's stable
argsort (a textbook stable sort) and bincount, and the invariants of the
bucketing."""
import json
import os

import numpy as np
import pytest

import moe_workloads as W
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLD, "permute_tiny.json")))
    ids = np.array(g["expert_ids"], dtype=np.int32)
    x = np.arange(g["T"] * 8, dtype=np.uint16).reshape(g["T"], 8)
    r = oracle.permute(x, ids, g["E"])
    np.testing.assert_array_equal(r["expert_counts"], g["expert_counts"])
    np.testing.assert_array_equal(r["expert_offsets"], g["expert_offsets"])
    np.testing.assert_array_equal(r["sorted_slot"], g["sorted_slot"])
    np.testing.assert_array_equal(r["row_of_slot"], np.array(g["row_of_slot"]))
    # row 0 holds token of slot 1 -> token 0; row 4 holds slot 0 -> token 0; row 2 slot 2 -> token 1
    np.testing.assert_array_equal(r["permuted"][2], x[1])


def _stable_sort_reference(ids, E):
    flat = ids.reshape(-1)
    real = (flat >= 0) & (flat < E)
    key = np.where(real, flat, E).astype(np.int64)
    order = np.argsort(key, kind="stable")
    n = int(real.sum())
    return order[:n], np.bincount(flat[real], minlength=E)


@pytest.mark.parametrize("T,K,E,seed,special", [
    (1, 1, 1, 0, 0), (7, 3, 5, 1, 0), (64, 2, 8, 2, 0), (333, 6, 64, 3, 0),
    (500, 8, 256, 4, 0), (129, 4, 16, 5, 4), (50, 16, 40, 6, 3),
])
def test_against_stable_argsort(T, K, E, seed, special):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E + special, size=(T, K)).astype(np.int32)
    if special:
        ids[0, 0] = -3  # negative ids are not real experts either
    x = W.normal_bf16(rng, (T, 24))
    r = oracle.permute(x, ids, E)
    order, counts = _stable_sort_reference(ids, E)
    n = order.size
    np.testing.assert_array_equal(r["expert_counts"], counts)
    assert r["expert_offsets"][0] == 0 and r["expert_offsets"][-1] == n
    np.testing.assert_array_equal(np.diff(r["expert_offsets"]), counts)
    np.testing.assert_array_equal(r["sorted_slot"][:n], order)
    assert np.all(r["sorted_slot"][n:] == -1)
    # invariants: counts plus non-real slots = T*K; the two maps are inverse
    flat = ids.reshape(-1)
    n_special = int(((flat < 0) | (flat >= E)).sum())
    assert int(r["expert_counts"].sum()) + n_special == T * K
    ros = r["row_of_slot"].reshape(-1)
    real = (flat >= 0) & (flat < E)
    assert np.all(ros[~real] == -1)
    np.testing.assert_array_equal(r["sorted_slot"][ros[real]], np.flatnonzero(real))
    np.testing.assert_array_equal(ros[r["sorted_slot"][:n]], np.arange(n))
    # permuted rows are bit copies of their token
    np.testing.assert_array_equal(r["permuted"][:n], x[order // K])


def test_empty_and_all_special():
    ids = np.full((5, 2), 9, dtype=np.int32)
    r = oracle.permute(np.zeros((5, 8), np.uint16), ids, 4)
    assert r["expert_offsets"][-1] == 0
    assert np.all(r["sorted_slot"] == -1) and np.all(r["row_of_slot"] == -1)
    r0 = oracle.permute(np.zeros((0, 8), np.uint16), np.zeros((0, 3), np.int32), 4)
    assert r0["expert_offsets"].tolist() == [0, 0, 0, 0, 0]


def test_combine_v2_example_ids():
    g = json.load(open(os.path.join(GOLD, "combine_v2_example_ids.json")))
    ids = np.array(g["expert_ids"], dtype=np.int32)
    E = g["moe_expert_num"]
    r = oracle.permute(np.zeros((8, 8), np.uint16), ids, E)
    # ids 32 (zero expert) and 33 (copy expert) appear 4 times: not routed to rows
    assert int(r["expert_counts"].sum()) == 64 - 4
    assert np.all(r["row_of_slot"][ids >= E] == -1)
    order, counts = _stable_sort_reference(ids, E)
    np.testing.assert_array_equal(r["sorted_slot"][:60], order)
