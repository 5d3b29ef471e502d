"""Parity at the full workload sizes, in the launch configuration the benchmark times.

Workloads are generated on the GPU: the dense-neighbourhood one (233,000 nodes, 115M edges,
602-d rows with stride 604, batches of 1024 seeds, fanouts [25, 10]), the mid-scale one
(2.45M nodes, 124M edges, 100-d, fanouts [15, 10, 5], super-batches of 8) and the large one
(111M nodes, 1.6B edges, int64 indptr, 128-d, 57 GB of features in HBM).  Whole batches are
compared with the oracle (bit-exact blocks and rows, means within 1e-5 * max|X|), with both
super-batch relabel modes, and with the super-batches of 16 the benchmark runs on the dense and
large workloads.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import compare_with_oracle

pytestmark = pytest.mark.gpu

gm = pytest.importorskip("graph_mini_pipeline_amd")


def _workload(name):
    cfg = synth.CONFIGS[name]
    dev = torch.device("cuda")
    g = synth.build_graph(cfg, device=dev)
    table = torch.empty(cfg.num_nodes, cfg.ld, dtype=torch.float32, device=dev)
    synth.make_features(cfg, table)
    order = synth.epoch_seed_order(cfg, 0, device=dev).contiguous()
    host = (g.indptr.cpu().numpy(), g.indices.cpu().numpy(), table.cpu().numpy(),
            order.cpu().numpy())
    return cfg, g, table, order, host


@pytest.fixture(scope="module")
def dense():
    return _workload("dense")


@pytest.fixture(scope="module")
def mid():
    return _workload("mid")


@pytest.fixture(scope="module")
def large():
    w = _workload("large")
    yield w
    del w
    torch.cuda.empty_cache()


def _run(cfg, g, table, order, batches, seed64, mode="auto", exact_rank=False):
    dg = gm.DeviceGraph(cfg.num_nodes, g.indptr, g.indices)
    fs = gm.gnn_feature_store_create(table, cfg.d)
    lo = batches[0] * cfg.batch
    hi = min(order.numel(), (batches[-1] + 1) * cfg.batch)
    ptr = [b * cfg.batch - lo for b in batches] + [hi - lo]
    outs = [gm.MinibatchOut(gm.gnn_capacity(ptr[j + 1] - ptr[j], cfg.fanouts, cfg.num_nodes),
                            cfg.d, cfg.ld) for j in range(len(batches))]
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, cfg.num_nodes)
    ws = torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes, len(batches)), dtype=torch.uint8,
                     device="cuda")
    gm.gnn_minibatch(dg, fs, order[lo:hi], ptr, cfg.fanouts, seed64, outs, ws,
                     gm.Options(superbatch=mode, exact_rank=exact_rank))
    assert gm.gnn_read_device_status(ws) == gm.GNN_OK
    return outs, ptr


@pytest.mark.parametrize("b", [0, 146])
def test_dense_single_batch(dense, b):
    cfg, g, table, order, (indptr, indices, x, order_h) = dense
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, b)
    outs, _ = _run(cfg, g, table, order, [b], seed64)
    seeds = order_h[b * cfg.batch:(b + 1) * cfg.batch]
    ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
    compare_with_oracle(outs[0], ref, cfg.d)


@pytest.mark.parametrize("mode", ["auto", "compact"])
def test_dense_superbatch_of_8(dense, mode):
    cfg, g, table, order, (indptr, indices, x, order_h) = dense
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 3)
    batches = list(range(24, 32))
    outs, ptr = _run(cfg, g, table, order, batches, seed64, mode)
    for j in (0, 5):
        b = batches[j]
        seeds = order_h[b * cfg.batch:(b + 1) * cfg.batch]
        ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
        compare_with_oracle(outs[j], ref, cfg.d)


def test_dense_superbatch_of_16(dense):
    # the benchmark's super-batch size on this workload
    cfg, g, table, order, (indptr, indices, x, order_h) = dense
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 1)
    batches = list(range(16, 32))
    outs, ptr = _run(cfg, g, table, order, batches, seed64)
    for j in (0, 15):
        b = batches[j]
        seeds = order_h[b * cfg.batch:(b + 1) * cfg.batch]
        ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
        compare_with_oracle(outs[j], ref, cfg.d)


def test_dense_superbatch_last_partial(dense):
    # the epoch's last super-batch of 8: batches 144..146, the last one short (496 seeds)
    cfg, g, table, order, (indptr, indices, x, order_h) = dense
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 18)
    batches = [144, 145, 146]
    outs, ptr = _run(cfg, g, table, order, batches, seed64)
    b = 146
    seeds = order_h[b * cfg.batch:]
    assert len(seeds) == 496
    ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
    compare_with_oracle(outs[2], ref, cfg.d)


@pytest.mark.parametrize("mode", ["auto", "compact"])
def test_mid_superbatch_of_8(mid, mode):
    cfg, g, table, order, (indptr, indices, x, order_h) = mid
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 0)
    batches = list(range(0, 8))
    outs, ptr = _run(cfg, g, table, order, batches, seed64, mode)
    for j in (0, 7):
        b = batches[j]
        seeds = order_h[b * cfg.batch:(b + 1) * cfg.batch]
        ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
        compare_with_oracle(outs[j], ref, cfg.d)


@pytest.mark.parametrize("mode,check", [("auto", (0, 7)), ("full", (3,))])
def test_large_superbatch_of_8(large, mode, check):
    cfg, g, table, order, (indptr, indices, x, order_h) = large
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 0)
    batches = list(range(0, 8))
    outs, ptr = _run(cfg, g, table, order, batches, seed64, mode)
    for j in check:
        b = batches[j]
        seeds = order_h[b * cfg.batch:(b + 1) * cfg.batch]
        ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
        compare_with_oracle(outs[j], ref, cfg.d)


def test_large_superbatch_of_16(large):
    # the benchmark's super-batch size on this workload
    cfg, g, table, order, (indptr, indices, x, order_h) = large
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 2)
    batches = list(range(32, 48))
    outs, ptr = _run(cfg, g, table, order, batches, seed64)
    for j in (2, 15):
        b = batches[j]
        seeds = order_h[b * cfg.batch:(b + 1) * cfg.batch]
        ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
        compare_with_oracle(outs[j], ref, cfg.d)


def test_large_single_batch(large):
    cfg, g, table, order, (indptr, indices, x, order_h) = large
    b = 100_000
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, b)
    outs, _ = _run(cfg, g, table, order, [b], seed64)
    seeds = order_h[b * cfg.batch:(b + 1) * cfg.batch]
    ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
    compare_with_oracle(outs[0], ref, cfg.d)


@pytest.mark.parametrize("wl", ["dense", "mid"])
def test_high_word_ranking_equals_exact_ranking_full_size(request, wl):
    # one super-batch of 16 (dense) or 8 (mid) sampled with the default selection and with every
    # node ranked by (key, position): identical blocks for every sub-batch
    cfg, g, table, order, _ = request.getfixturevalue(wl)
    G = 16 if wl == "dense" else 8
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 3)
    batches = list(range(3 * G, 4 * G))
    fast, _ = _run(cfg, g, table, order, batches, seed64)
    exact, _ = _run(cfg, g, table, order, batches, seed64, exact_rank=True)
    for a, b in zip(fast, exact):
        for ha, hb in zip(a.blocks.host(), b.blocks.host()):
            for u, v in zip(ha, hb):
                assert np.array_equal(u, v)


def _headline_parity(workload, steps, G, rounds, label):
    """Sub-batches of `steps` issued in the benchmark's headline layout (three streams, each with
    its own workspace and outputs, super-batches of G) against the oracle, which runs on host
    threads while the GPU works; every block array and X bit for bit, every h within tolerance."""
    import sys
    from tests.gpu_util import headline_layout, oracle_pool
    cfg, g, table, order, (indptr, indices, x, order_h) = workload
    dg = gm.DeviceGraph(cfg.num_nodes, g.indptr, g.indices)
    fs = gm.gnn_feature_store_create(table, cfg.d)
    n_batches = (len(order_h) + cfg.batch - 1) // cfg.batch
    bs = [b for st in steps for b in range(st * G, min(st * G + G, n_batches))]
    jobs = [(b, order_h[b * cfg.batch:(b + 1) * cfg.batch], cfg.fanouts,
             gm.gnn_batch_seed(cfg.rng_seed, b // G)) for b in bs]
    ex, futs = oracle_pool(indptr, indices, x, cfg.d, jobs)
    seen = []
    try:
        for st, b, seed64, out in headline_layout(cfg, dg, fs, order, steps, G, rounds=rounds):
            compare_with_oracle(out, futs.pop(b).result(), cfg.d)
            seen.append(b)
            if len(seen) % 16 == 0:
                print(f"[{label}] {len(seen)}/{len(bs)} sub-batches equal the oracle",
                      file=sys.stderr, flush=True)
    finally:
        ex.shutdown(cancel_futures=True)
        torch.cuda.empty_cache()
    assert sorted(seen) == sorted(bs)


@pytest.mark.timeout(1200)
def test_dense_full_epoch_in_headline_layout(dense):
    """All 147 batches of the epoch (146 of 1024 seeds and one of 496): ten super-batches of 16
    on three streams, two per stream in flight before the host synchronises (GARDEN Sec. IV.D:
    each mini-batch keeps its own logical result inside a super-batch)."""
    _headline_parity(dense, range(10), 16, 2, "dense epoch")


@pytest.mark.timeout(1200)
def test_large_three_streams_in_headline_layout(large):
    """Three super-batches of 16 (48 mini-batches) at once on three streams, as the headline runs
    them on the 111M-node graph; every sub-batch against the oracle."""
    _headline_parity(large, range(3), 16, 1, "large")
