"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each pin is independent of the oracle's own code path: published SplitMix64 outputs, brute force
with Python's sort, a textbook BFS, numpy's unique, dense matrix products, exact rationals,
hand-derived results and sampling statistics.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import helpers as H

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


# ---- hash ------------------------------------------------------------------------------------

def test_splitmix_published_outputs():
    seed, expected = H.read_golden_splitmix()
    assert oracle.splitmix_stream(seed, len(expected)) == expected


def test_edge_keys_are_the_node_stream():
    # key of position j is output j+1 of the SplitMix64 stream started at the node seed
    for state in (0, 1234567, M64, 0xDEADBEEFCAFEF00D):
        stream = oracle.splitmix_stream(state, 40)
        assert [oracle.edge_key(state, j) for j in range(40)] == stream


def test_seed_chain_is_stream_outputs():
    for r in (0, 7, 1234567):
        s = oracle.splitmix_stream(r, 6)
        assert [oracle.batch_seed(r, b) for b in range(6)] == s
        assert [oracle.hop_seed(r, l) for l in range(1, 7)] == s
    # node seed: the output function applied to hop_seed xor v; output of a stream whose state is
    # one step before that value
    for hs in (3, 1234567, M64):
        for v in (0, 1, 77, 2**31 - 1):
            z = hs ^ v
            assert oracle.node_seed(hs, v) == oracle.splitmix_stream((z - GAMMA) & M64, 1)[0]


# ---- sampling --------------------------------------------------------------------------------

def brute_positions(ns: int, deg: int, k: int):
    keys = oracle.splitmix_stream(ns, deg)
    if deg <= k:
        return list(range(deg))
    order = sorted(range(deg), key=lambda j: (keys[j], j))
    return sorted(order[:k])


@pytest.mark.parametrize("deg,k", [(0, 1), (1, 1), (5, 5), (6, 5), (5, 6), (7, 3), (64, 10),
                                   (200, 25), (1000, 15), (31, 30)])
def test_select_positions_brute(deg, k):
    for ns in (1, 99, 1234567, M64):
        got = oracle.select_positions(ns, deg, k).tolist()
        assert got == brute_positions(ns, deg, k)
        assert len(got) == min(deg, k)
        assert len(set(got)) == len(got)
        assert got == sorted(got)


def test_select_positions_nested_in_k():
    # bottom-k: the k-sample is contained in the (k+1)-sample of the same keys
    for ns in range(20):
        prev = set()
        for k in range(1, 30):
            cur = set(oracle.select_positions(ns * 7919 + 1, 30, k).tolist())
            assert prev <= cur and len(cur) == min(30, k)
            prev = cur


def _check_block(indptr, indices, front, k, seed64, hop, blk_indptr, gid):
    hs = oracle.hop_seed(seed64, hop)
    assert blk_indptr[0] == 0
    for i, v in enumerate(front):
        s, e = int(indptr[v]), int(indptr[v + 1])
        row = indices[s:e]
        pos = brute_positions(oracle.node_seed(hs, int(v)), e - s, k)
        got = gid[blk_indptr[i]:blk_indptr[i + 1]]
        assert got.tolist() == [int(row[j]) for j in pos]
        if e - s <= k:
            assert got.tolist() == row.tolist()   # full node: the whole row, in CSR order


@pytest.mark.parametrize("graph", ["star", "path", "complete", "hand", "random"])
def test_sample_hop_hand_graphs(graph):
    if graph == "star":
        indptr, indices = H.star(30)
    elif graph == "path":
        indptr, indices = H.path(12)
    elif graph == "complete":
        indptr, indices = H.complete(6)
    elif graph == "hand":
        indptr, indices, _, _ = H.read_hand_graph()
    else:
        indptr, indices = H.random_csr(300, 12, seed=5, indptr_dtype=np.int64)
    n = indptr.shape[0] - 1
    front = np.arange(n, dtype=np.int32)[::-1].copy()
    for k in (1, 2, 3, 5, 6, 25):
        for seed64 in (0, 11):
            for hop in (1, 2):
                bi, gid = oracle.sample_hop(indptr, indices, front, k, seed64, hop)
                _check_block(indptr, indices, front, k, seed64, hop, bi, gid)


def test_sampling_inclusion_is_uniform():
    # star centre with D in-neighbours, k drawn: every neighbour is included with prob k/D
    D, k, S = 20, 5, 12000
    indptr, indices = H.star(D)
    counts = np.zeros(D + 1, dtype=np.int64)
    for b in range(S):
        _, gid = oracle.sample_hop(indptr, indices, np.array([0], np.int32), k,
                                   oracle.batch_seed(0, b), 1)
        assert len(set(gid.tolist())) == k
        counts[gid] += 1
    p = k / D
    z = (counts[1:] - S * p) / np.sqrt(S * p * (1 - p))
    assert np.abs(z).max() < 4.5


def test_sampling_pairs_are_uniform():
    # degree 6, fanout 2: each of the 15 pairs has probability 1/15 (chi-square, 14 dof)
    D, k, S = 6, 2, 15000
    counts = {}
    for b in range(S):
        pos = tuple(oracle.select_positions(oracle.batch_seed(1, b), D, k).tolist())
        counts[pos] = counts.get(pos, 0) + 1
    assert len(counts) == 15
    obs = np.array(list(counts.values()), dtype=np.float64)
    chi2 = ((obs - S / 15) ** 2 / (S / 15)).sum()
    assert chi2 < 45.0   # P(chi2_14 > 45) ~ 4e-5


@pytest.mark.parametrize("hops", [1, 2, 3])
def test_full_fanout_is_bfs(hops):
    indptr, indices = H.random_csr(400, 4, seed=hops)
    deg = np.diff(indptr)
    seeds = np.array([3, 17, 250, 399, 0], dtype=np.int32)
    blocks = oracle.sample_khop(indptr, indices, seeds, [int(deg.max())] * hops, 123)
    for l, layer in enumerate(H.bfs_layers(indptr, indices, seeds, hops)):
        assert blocks[l].nodes.tolist() == layer.tolist()


# ---- relabel ---------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_relabel_matches_numpy_unique(seed):
    rng = np.random.default_rng(seed)
    front = rng.choice(5000, size=300, replace=False).astype(np.int32)
    gid = rng.integers(0, 5000, size=2000).astype(np.int32)
    uniq, lid, dst = oracle.relabel(front, gid)
    u, inv = np.unique(np.concatenate([front, gid]), return_inverse=True)
    assert uniq.tolist() == u.tolist()
    assert dst.tolist() == inv[:300].tolist()
    assert lid.tolist() == inv[300:].tolist()
    assert np.all(np.diff(uniq) > 0)
    assert np.array_equal(uniq[lid], gid) and np.array_equal(uniq[dst], front)


def test_relabel_empty_and_degenerate():
    uniq, lid, dst = oracle.relabel(np.zeros(0, np.int32), np.zeros(0, np.int32))
    assert uniq.size == 0 and lid.size == 0 and dst.size == 0
    uniq, lid, dst = oracle.relabel(np.array([5], np.int32), np.array([5, 5, 5], np.int32))
    assert uniq.tolist() == [5] and lid.tolist() == [0, 0, 0] and dst.tolist() == [0]


# ---- gather ----------------------------------------------------------------------------------

def test_gather_is_byte_copy():
    rng = np.random.default_rng(3)
    table = rng.standard_normal((1000, 13)).astype(np.float32)
    table[5, 2] = np.float32(-0.0)
    table[7, 1] = np.float32(np.nan)
    ids = rng.integers(0, 1000, size=500).astype(np.int32)
    ids[:3] = [5, 7, 999]
    out = oracle.gather(table, ids, 11)
    assert np.array_equal(out.view(np.uint32), table[ids, :11].view(np.uint32))


# ---- mean ------------------------------------------------------------------------------------

def test_mean_exact_rationals():
    rng = np.random.default_rng(4)
    src = rng.uniform(-1, 1, size=(50, 5)).astype(np.float32)
    counts = rng.integers(0, 9, size=40)
    blk_indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    lid = rng.integers(0, 50, size=int(counts.sum())).astype(np.int32)
    out = oracle.mean_aggregate(blk_indptr, lid, src)
    for i in range(40):
        es = range(blk_indptr[i], blk_indptr[i + 1])
        for t in range(5):
            if len(es) == 0:
                assert out[i, t] == 0.0
                continue
            exact = sum(Fraction(float(src[lid[e], t])) for e in es) / len(es)
            err = abs(Fraction(float(out[i, t])) - exact)
            ulp = np.spacing(np.float32(abs(float(exact)))).astype(np.float64)
            assert err <= Fraction(float(ulp))


def test_mean_is_row_normalised_adjacency():
    indptr, indices = H.random_csr(120, 6, seed=9)
    n = 120
    x = np.random.default_rng(1).standard_normal((n, 7)).astype(np.float32)
    P = H.mean_operator(indptr, indices, n)
    seeds = np.arange(0, n, 3, dtype=np.int32)
    maxdeg = int(np.diff(indptr).max())
    for K in (1, 2, 3):
        mb = oracle.minibatch(indptr, indices, x, seeds, [maxdeg] * K, 5)
        ref = np.linalg.matrix_power(P, K) @ x.astype(np.float64)
        np.testing.assert_allclose(mb.h[0], ref[seeds], rtol=0, atol=2e-6 * K)


# ---- whole path on the hand-built graph ------------------------------------------------------

def _frac_rows(vals, d):
    return np.array([float(v) for v in vals], dtype=np.float64).reshape(-1, d)


def test_hand_graph_golden():
    indptr, indices, x, cases = H.read_hand_graph()
    a = cases["A"]
    mb = oracle.minibatch(indptr, indices, x, np.array(a["seeds"], np.int32), a["fanouts"], 42)
    assert mb.blocks[0].nodes.tolist() == a["V1"]
    assert mb.blocks[0].gid.tolist() == a["gid"]
    assert mb.blocks[0].indptr.tolist() == a["indptr"]
    np.testing.assert_allclose(mb.h[0], _frac_rows(a["h0"], 2), rtol=0, atol=1e-6)
    assert np.array_equal(mb.x, x[mb.blocks[0].nodes])
    b = cases["B"]
    mb = oracle.minibatch(indptr, indices, x, np.array(b["seeds"], np.int32), b["fanouts"], 42)
    assert mb.blocks[0].nodes.tolist() == b["V1"]
    assert mb.blocks[1].nodes.tolist() == b["V2"]
    np.testing.assert_allclose(mb.h[1], _frac_rows(b["h1"], 2), rtol=0, atol=1e-6)
    np.testing.assert_allclose(mb.h[0], _frac_rows(b["h0"], 2), rtol=0, atol=1e-6)


def test_invalid_seeds_rejected():
    indptr, indices = H.path(5)
    with pytest.raises(RuntimeError):
        oracle.sample_khop(indptr, indices, np.array([1, 1], np.int32), [2], 0)
    with pytest.raises(RuntimeError):
        oracle.sample_khop(indptr, indices, np.array([5], np.int32), [2], 0)


def test_superbatch_is_independent_runs():
    indptr, indices = H.random_csr(200, 8, seed=2)
    x = np.random.default_rng(0).standard_normal((200, 3)).astype(np.float32)
    seeds = np.arange(0, 60, dtype=np.int32)
    ptr = [0, 20, 45, 60]
    sb = oracle.superbatch(indptr, indices, x, seeds, ptr, [4, 3], 77)
    for g in range(3):
        one = oracle.minibatch(indptr, indices, x, seeds[ptr[g]:ptr[g + 1]], [4, 3], 77)
        assert np.array_equal(sb[g].h[0], one.h[0])
        for a, b in zip(sb[g].blocks, one.blocks):
            assert np.array_equal(a.gid, b.gid) and np.array_equal(a.nodes, b.nodes)


# ---- GraphSAGE-mean layer --------------------------------------------------------------------

def _random_block(rng, n_dst, n_src, max_c):
    counts = rng.integers(0, max_c + 1, size=n_dst)
    counts[:2] = 0   # rows without sampled neighbours
    blk_indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    lid = rng.integers(0, n_src, size=int(counts.sum())).astype(np.int32)
    dst_lid = rng.permutation(n_src)[:n_dst].astype(np.int32)
    return blk_indptr, lid, dst_lid


@pytest.mark.parametrize("relu", [False, True])
def test_sage_layer_exact_rationals(relu):
    """Each output against exact rational arithmetic: [self || mean] @ W + bias, then ReLU."""
    rng = np.random.default_rng(21)
    n_dst, n_src, d, d_out = 9, 14, 3, 5
    blk_indptr, lid, dst_lid = _random_block(rng, n_dst, n_src, 6)
    src = rng.uniform(-2, 2, size=(n_src, d)).astype(np.float32)
    W = rng.uniform(-1, 1, size=(2 * d, d_out)).astype(np.float32)
    b = rng.uniform(-1, 1, size=d_out).astype(np.float32)
    out, scale = oracle.sage_layer(blk_indptr, lid, dst_lid, src, W, b, relu, with_scale=True)
    for i in range(n_dst):
        es = range(blk_indptr[i], blk_indptr[i + 1])
        a = [Fraction(float(src[dst_lid[i], t])) for t in range(d)]
        for t in range(d):
            a.append(sum((Fraction(float(src[lid[e], t])) for e in es), Fraction(0)) / len(es)
                     if len(es) else Fraction(0))
        for n in range(d_out):
            lin = sum((a[k] * Fraction(float(W[k, n])) for k in range(2 * d)), Fraction(float(b[n])))
            exact = max(lin, Fraction(0)) if relu else lin
            mag = sum((abs(a[k]) * abs(Fraction(float(W[k, n]))) for k in range(2 * d)),
                      abs(Fraction(float(b[n]))))
            tol = Fraction(2.0 ** -50) * mag
            assert abs(Fraction(float(out[i, n])) - exact) <= tol, (i, n)
            assert abs(Fraction(float(scale[i, n])) - mag) <= tol, (i, n)


def test_sage_layer_is_dense_algebra():
    """relu(A @ W + b) with A = [X[dst_lid] | P X], P the row-normalised block adjacency."""
    rng = np.random.default_rng(22)
    n_dst, n_src, d, d_out = 40, 70, 6, 11
    blk_indptr, lid, dst_lid = _random_block(rng, n_dst, n_src, 9)
    x = rng.standard_normal((n_src, d)).astype(np.float32)
    W = rng.standard_normal((2 * d, d_out)).astype(np.float32)
    b = rng.standard_normal(d_out).astype(np.float32)
    P = np.zeros((n_dst, n_src))
    for i in range(n_dst):
        c = blk_indptr[i + 1] - blk_indptr[i]
        for e in range(blk_indptr[i], blk_indptr[i + 1]):
            P[i, lid[e]] += 1.0 / c
    A = np.concatenate([x[dst_lid].astype(np.float64), P @ x.astype(np.float64)], axis=1)
    ref = A @ W.astype(np.float64) + b
    np.testing.assert_allclose(oracle.sage_layer(blk_indptr, lid, dst_lid, x, W, b, False), ref,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.sage_layer(blk_indptr, lid, dst_lid, x, W, b, True),
                               np.maximum(ref, 0.0), rtol=1e-12, atol=1e-12)


def test_sage_layer_special_cases():
    """Identity halves of W give the node's own row or the mean; W = 0 gives relu(bias)."""
    rng = np.random.default_rng(23)
    n_dst, n_src, d = 30, 50, 4
    blk_indptr, lid, dst_lid = _random_block(rng, n_dst, n_src, 7)
    x = rng.standard_normal((n_src, d)).astype(np.float32)
    I, Z = np.eye(d, dtype=np.float32), np.zeros((d, d), np.float32)
    own = oracle.sage_layer(blk_indptr, lid, dst_lid, x, np.concatenate([I, Z]), relu=False)
    assert np.array_equal(own, x[dst_lid].astype(np.float64))
    mean = oracle.sage_layer(blk_indptr, lid, dst_lid, x, np.concatenate([Z, I]), relu=False)
    m32 = oracle.mean_aggregate(blk_indptr, lid, x)
    assert np.array_equal(mean.astype(np.float32), m32)   # the float mean rounds the double one
    assert np.all(mean[:2] == 0.0)
    b = np.array([1.5, -2.0, 0.0, 3.25], np.float32)
    only_b = oracle.sage_layer(blk_indptr, lid, dst_lid, x, np.zeros((2 * d, 4), np.float32), b)
    assert np.array_equal(only_b, np.tile(np.maximum(b, 0).astype(np.float64), (n_dst, 1)))
