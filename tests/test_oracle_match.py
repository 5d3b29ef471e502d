"""Pins of the oracle's Match and Greedy Reorder (FastGL, "The idea" and "What it costs"), and the
library's host-side greedy order against it (host code, no GPU)."""
import math

import numpy as np
import pytest

import oracle


def multiples(p, N):
    return np.arange(0, N, p, dtype=np.int32)


def test_overlap_closed_form_of_multiples():
    # multiples of p and of q below N share exactly the multiples of lcm(p, q): floor((N-1)/lcm)+1
    N = 10_007
    ps = [2, 3, 5, 6, 7, 10, 11]
    m = oracle.batch_overlap([multiples(p, N) for p in ps])
    for a, p in enumerate(ps):
        for b, q in enumerate(ps):
            l = p * q // math.gcd(p, q)
            assert m[a, b] == (N - 1) // l + 1


def test_overlap_special_cases():
    e = np.zeros(0, np.int32)
    m = oracle.batch_overlap([e, np.array([1, 5, 9], np.int32), np.array([5], np.int32), e])
    assert m.tolist() == [[0, 0, 0, 0], [0, 3, 1, 0], [0, 1, 1, 0], [0, 0, 0, 0]]


def test_match_positions_special_cases():
    prev = np.array([2, 4, 8, 16], np.int32)
    assert oracle.match_positions([16, 3, 2, 8, 9], prev).tolist() == [3, -1, 0, 2, -1]
    assert oracle.match_positions([], prev).tolist() == []
    assert oracle.match_positions([1, 2], np.zeros(0, np.int32)).tolist() == [-1, -1]


def test_greedy_order_hand_worked():
    # from batch 0: its largest overlap is batch 2 (4); from 2, batch 1 (2 > 1); then 3
    m = np.array([[5, 1, 4, 0], [1, 6, 2, 3], [4, 2, 7, 1], [0, 3, 1, 4]])
    assert oracle.greedy_order(m, 0) == [0, 2, 1, 3]
    # from batch 3: batch 1 (3); from 1, batch 2 (2 > 1); then 0
    assert oracle.greedy_order(m, 3) == [3, 1, 2, 0]


def test_greedy_order_ties_take_the_smaller_index():
    m = np.full((5, 5), 7, dtype=np.int64)
    assert oracle.greedy_order(m, 2) == [2, 0, 1, 3, 4]


def test_greedy_order_follows_a_chain():
    # overlaps only between neighbours of a hidden chain 4-1-3-0-2: the order walks the chain
    chain = [4, 1, 3, 0, 2]
    m = np.zeros((5, 5), dtype=np.int64)
    for x, y in zip(chain, chain[1:]):
        m[x, y] = m[y, x] = 10
    assert oracle.greedy_order(m, 4) == chain


def test_greedy_order_is_a_permutation_starting_at_first():
    rng = np.random.default_rng(5)
    for B in (1, 2, 7, 16):
        m = rng.integers(0, 100, size=(B, B))
        m = m + m.T
        for first in range(B):
            o = oracle.greedy_order(m, first)
            assert o[0] == first and sorted(o) == list(range(B))


def test_library_greedy_order_matches_the_oracle():
    gm = pytest.importorskip("graph_mini_pipeline_amd")
    rng = np.random.default_rng(9)
    for B in (1, 3, 8, 16):
        for trial in range(20):
            m = rng.integers(0, 6, size=(B, B))    # small values: many ties
            m = m + m.T
            first = int(rng.integers(0, B))
            assert gm.gnn_greedy_order(m, first) == oracle.greedy_order(m, first)
    with pytest.raises(Exception):
        gm.gnn_greedy_order(np.zeros((3, 3), np.int64), 3)
