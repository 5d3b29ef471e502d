"""Pins of the oracle's Dynamic-Cache policy (GARDEN Sec. IV.B, eq. (5)-(6)) against a schedule
worked by hand, closed forms of the decayed count, and brute force over every k-subset."""
import itertools
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dyn_cache_schedule.txt")


def _scenarios():
    runs, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, *rest = line.split()
            if head == "scenario":
                cur = {"max_refreshes": int(rest[0]), "events": []}
                runs.append(cur)
            elif head in ("observe", "update"):
                cur["events"].append([head, [int(t) for t in rest], None, None])
            elif head == "score":
                cur["events"][-1][2] = np.array([float(t) for t in rest])
            elif head == "members":
                cur["events"][-1][3] = [] if rest == ["-"] else [int(t) for t in rest]
    return runs


@pytest.mark.parametrize("run", _scenarios(), ids=lambda r: f"max_refreshes={r['max_refreshes']}")
def test_schedule_worked_by_hand(run):
    dc = oracle.DynCache(5, [3], 0.5, 1, 2, run["max_refreshes"])
    for kind, ids, score, members in run["events"]:
        if kind == "observe":
            dc.observe(np.array(ids, dtype=np.int32))
        else:
            dc.update()
        np.testing.assert_array_equal(dc.score, score)   # binary fractions: exact
        assert dc.members.tolist() == members


def test_every_step_gives_the_geometric_series():
    g, T = 0.9, 60
    s = np.zeros(3)
    for _ in range(T):
        oracle.dyn_ewma_step(s, g, [1], None)
    assert s[1] == pytest.approx((1 - g ** T) / (1 - g), rel=1e-13)
    assert s[0] == 0 and s[2] == 0


def test_one_access_decays_as_a_power():
    g = 0.8
    s = np.zeros(4)
    oracle.dyn_ewma_step(s, g, [2, 2, 2], None)   # three occurrences in one mini-batch
    for _ in range(25):
        oracle.dyn_ewma_step(s, g, [], None)
    assert s[2] == pytest.approx(3 * g ** 25, rel=1e-13)


def test_static_rows_are_never_scored():
    s = np.zeros(6)
    st = np.array([1, 0, 0, 1, 0, 0], dtype=np.uint8)
    rng = np.random.default_rng(3)
    for _ in range(10):
        oracle.dyn_ewma_step(s, 0.7, rng.integers(0, 6, 20), st)
    assert s[0] == 0 and s[3] == 0
    assert (s[[1, 2, 4, 5]] > 0).all()
    assert not set(oracle.dyn_topk(s, 6).tolist()) & {0, 3}


def _dominates(s, a, b):
    return s[a] > s[b] or (s[a] == s[b] and a < b)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("k", [0, 1, 3, 5, 9])
def test_topk_is_the_one_subset_that_dominates_the_rest(seed, k):
    rng = np.random.default_rng(seed)
    n = 8
    s = rng.integers(0, 4, n).astype(np.float64) / 2   # many ties and zeros
    pos = [v for v in range(n) if s[v] > 0]
    m = min(k, len(pos))
    winners = [set(c) for c in itertools.combinations(pos, m)
               if all(_dominates(s, a, b) for a in c for b in pos if b not in c)]
    assert len(winners) == 1
    assert set(oracle.dyn_topk(s, k).tolist()) == winners[0]


def test_topk_output_is_ascending_and_bounded():
    s = np.array([0.0, 3.0, 1.0, 3.0, 0.5, 0.0, 2.0])
    out = oracle.dyn_topk(s, 3)
    assert out.tolist() == [1, 3, 6]
    assert oracle.dyn_topk(s, 100).tolist() == [1, 2, 3, 4, 6]
    assert oracle.dyn_topk(np.zeros(4), 2).tolist() == []


def test_refresh_waits_for_t_update_mini_batches():
    dc = oracle.DynCache(10, [], 0.5, 2, 3)
    for i in range(2):
        dc.observe([i])
        assert not dc.update()
    dc.observe([5])
    assert dc.update() and dc.refreshes == 1
    assert not dc.update()   # nothing observed since
