"""Parity of the HIP path (through the C ABI) with the oracle, on small graphs and edge cases.

Bit-exact: sampled blocks, relabel maps, gathered rows.  Aggregation: max |err| <= 1e-5 * max|X|
per layer (fp32 sums of at most `fanout` terms against a double-accumulated reference).
"""
import numpy as np
import pytest
import torch

import synth
import oracle
from tests import helpers as H
from tests.gpu_util import compare_with_oracle, device_graph, device_table, run_minibatch

pytestmark = pytest.mark.gpu

gm = pytest.importorskip("graph_mini_pipeline_amd")


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    g = synth.build_graph(cfg)
    x = torch.empty(cfg.num_nodes, cfg.d, dtype=torch.float32)
    synth.make_features(cfg, x)
    order = synth.epoch_seed_order(cfg)
    return cfg, g.indptr.numpy(), g.indices.numpy(), x.numpy(), order.numpy()


def _store(x, ld=None):
    n, d = x.shape
    ld = ld or (d + 3) // 4 * 4
    return gm.gnn_feature_store_create(device_table(x, ld), d)


@pytest.mark.parametrize("batch", [0, 1, 2, 38])
def test_tiny_pipeline_matches_oracle(tiny, batch):
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    fs = _store(x)
    seeds = order[batch * cfg.batch:(batch + 1) * cfg.batch]
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, batch)
    outs, st = run_minibatch(dg, fs, seeds, cfg.fanouts, seed64)
    assert st == gm.GNN_OK
    ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64)
    compare_with_oracle(outs[0], ref, cfg.d)


@pytest.mark.parametrize("G,rounds", [(16, 2), (1, 3)])
def test_tiny_every_batch_in_headline_layout(tiny, G, rounds):
    """All 40 batches of the workload, issued as the benchmark's headline issues them (super-batches
    of G on three streams, each with its own workspace and outputs, several in flight at once);
    every sub-batch equals the oracle's separate run with its super-batch's seed (GARDEN Sec.
    IV.D: each mini-batch keeps its own logical result inside a super-batch)."""
    from tests.gpu_util import headline_layout, oracle_pool
    cfg, indptr, indices, x, order = tiny
    n_batches = (len(order) + cfg.batch - 1) // cfg.batch
    assert n_batches == 40
    dg = device_graph(indptr, indices)
    fs = _store(x)
    order_d = torch.from_numpy(order).cuda()
    n_super = (n_batches + G - 1) // G
    jobs = [(b, order[b * cfg.batch:(b + 1) * cfg.batch], cfg.fanouts,
             gm.gnn_batch_seed(cfg.rng_seed, b // G)) for b in range(n_batches)]
    ex, futs = oracle_pool(indptr, indices, x, cfg.d, jobs)
    seen = []
    try:
        for st, b, seed64, out in headline_layout(cfg, dg, fs, order_d, range(n_super), G,
                                                  rounds=rounds):
            compare_with_oracle(out, futs[b].result(), cfg.d)
            seen.append(b)
    finally:
        ex.shutdown(cancel_futures=True)
    assert sorted(seen) == list(range(n_batches))


@pytest.mark.parametrize("fanouts", [[5, 10], [5, 10, 15], [5, 5, 10, 10]])
@pytest.mark.parametrize("mode", ["full", "compact"])
def test_fanout_patterns(tiny, fanouts, mode):
    """GARDEN's fanout-pattern sweep (two to four hops), in super-batches of three overlapping
    sub-batches, in both relabel modes."""
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    fs = _store(x)
    seeds = np.concatenate([order[:300], order[200:450], order[100:180]])   # overlapping
    ptr = [0, 300, 550, 630]
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 5)
    opts = gm.Options(superbatch=mode)
    outs, st = run_minibatch(dg, fs, seeds, fanouts, seed64, opts, group_ptr=ptr)
    assert st == gm.GNN_OK
    for g in range(3):
        ref = oracle.minibatch(indptr, indices, x, seeds[ptr[g]:ptr[g + 1]], fanouts, seed64)
        compare_with_oracle(outs[g], ref, cfg.d)


@pytest.mark.parametrize("mode", ["full", "compact"])
def test_max_hops(tiny, mode):
    """GNN_MAX_HOPS = 8 hops (the last ones saturate the 10k-node graph), two sub-batches."""
    cfg, indptr, indices, x, order = tiny
    fanouts = [3, 2, 2, 2, 2, 2, 2, 2]
    assert len(fanouts) == 8
    dg = device_graph(indptr, indices)
    fs = _store(x)
    seeds = order[:96]
    ptr = [0, 40, 96]
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 9)
    outs, st = run_minibatch(dg, fs, seeds, fanouts, seed64, gm.Options(superbatch=mode),
                             group_ptr=ptr)
    assert st == gm.GNN_OK
    for g in range(2):
        ref = oracle.minibatch(indptr, indices, x, seeds[ptr[g]:ptr[g + 1]], fanouts, seed64)
        compare_with_oracle(outs[g], ref, cfg.d)


@pytest.mark.parametrize("group_max,wave_max", [(1, 1), (8, 32), (16, 100), (256, 4096), (256, 16384),
                                                (100000, 100000)])
def test_degree_classes_do_not_change_results(tiny, group_max, wave_max):
    # (1,1) sends every random node to the workgroup class, (100000,100000) to the 16-lane class
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    fs = _store(x)
    seeds = order[:cfg.batch]
    seed64 = gm.gnn_batch_seed(7, 0)
    outs, st = run_minibatch(dg, fs, seeds, [25, 10, 3], seed64,
                             gm.Options(group_max_deg=group_max, wave_max_deg=wave_max))
    assert st == gm.GNN_OK
    ref = oracle.minibatch(indptr, indices, x, seeds, [25, 10, 3], seed64)
    compare_with_oracle(outs[0], ref, cfg.d)


@pytest.mark.parametrize("graph", ["star", "bigstar", "path", "complete", "hand", "random64"])
@pytest.mark.parametrize("fanouts", [[1], [3, 3], [5, 2, 7], [25, 10]])
def test_hand_graphs(graph, fanouts):
    if graph == "star":
        indptr, indices = H.star(40)
    elif graph == "bigstar":
        indptr, indices = H.star(20000)       # a hub far above every class bound
    elif graph == "path":
        indptr, indices = H.path(50)
    elif graph == "complete":
        indptr, indices = H.complete(30)
    elif graph == "hand":
        indptr, indices, _, _ = H.read_hand_graph()
    else:
        indptr, indices = H.random_csr(2000, 40, seed=3, max_deg=600, indptr_dtype=np.int64)
    n = indptr.shape[0] - 1
    x = np.random.default_rng(n).standard_normal((n, 6)).astype(np.float32)
    dg = device_graph(indptr, indices)
    fs = _store(x, ld=6)            # ld = d = 6: the unaligned (scalar) gather/mean path
    seeds = np.arange(0, n, max(1, n // 37), dtype=np.int32)[::-1].copy()
    for seed64 in (0, 99):
        outs, st = run_minibatch(dg, fs, seeds, fanouts, seed64)
        assert st == gm.GNN_OK
        ref = oracle.minibatch(indptr, indices, x, seeds, fanouts, seed64)
        compare_with_oracle(outs[0], ref, 6)


def test_empty_seeds(tiny):
    cfg, indptr, indices, x, order = tiny
    outs, st = run_minibatch(device_graph(indptr, indices), _store(x), order[:0], [4, 2], 1)
    assert st == gm.GNN_OK
    assert outs[0].blocks.counts.cpu().tolist() == [0, 0, 0, 0]
    assert outs[0].blocks.indptr[0][0].item() == 0


def test_isolated_seed_and_zero_degree():
    indptr, indices = H.csr_from_rows([[], [0], [], [1, 2]])
    x = np.arange(8, dtype=np.float32).reshape(4, 2)
    outs, st = run_minibatch(device_graph(indptr, indices), _store(x, 4),
                             np.array([0, 2], np.int32), [3], 5)
    assert st == gm.GNN_OK
    ref = oracle.minibatch(indptr, indices, x, np.array([0, 2], np.int32), [3], 5)
    compare_with_oracle(outs[0], ref, 2)
    assert np.all(outs[0].h[0][:2, :2].cpu().numpy() == 0)


def test_duplicate_seed_reported(tiny):
    cfg, indptr, indices, x, order = tiny
    seeds = np.array([5, 17, 5], np.int32)
    _, st = run_minibatch(device_graph(indptr, indices), _store(x), seeds, [3], 1)
    assert st == gm.GNN_ERR_INVALID_ARG


def test_out_of_range_seed_reported(tiny):
    cfg, indptr, indices, x, order = tiny
    seeds = np.array([5, cfg.num_nodes, 7], np.int32)
    _, st = run_minibatch(device_graph(indptr, indices), _store(x), seeds, [3, 2], 1)
    assert st == gm.GNN_ERR_OUT_OF_RANGE


def test_capacity_overflow_reported(tiny):
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    seeds = torch.from_numpy(order[:64].copy()).cuda()
    caps = gm.gnn_capacity(64, [10, 5], cfg.num_nodes)
    caps.edges[1] = 7          # far below what hop 2 samples
    blocks = gm.Blocks(caps)
    ws = torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes), dtype=torch.uint8, device="cuda")
    gm.gnn_sample_khop(dg, seeds, [10, 5], 3, blocks, ws)
    assert gm.gnn_read_device_status(ws) == gm.GNN_ERR_CAPACITY


def test_sync_flag_returns_device_status(tiny):
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    seeds = torch.tensor([3, 3], dtype=torch.int32, device="cuda")
    caps = gm.gnn_capacity(2, [4], cfg.num_nodes)
    blocks = gm.Blocks(caps)
    ws = torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes), dtype=torch.uint8, device="cuda")
    with pytest.raises(gm.GnnError) as e:
        gm.gnn_sample_khop(dg, seeds, [4], 3, blocks, ws, gm.Options(sync=True))
    assert e.value.status == gm.GNN_ERR_INVALID_ARG


def test_sample_khop_alone_matches_oracle(tiny):
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    seeds = order[300:812]
    caps = gm.gnn_capacity(len(seeds), [8, 4, 2], cfg.num_nodes)
    blocks = gm.Blocks(caps)
    ws = torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes), dtype=torch.uint8, device="cuda")
    gm.gnn_sample_khop(dg, torch.from_numpy(seeds.copy()).cuda(), [8, 4, 2], 12345, blocks, ws)
    assert gm.gnn_read_device_status(ws) == gm.GNN_OK
    ref = oracle.sample_khop(indptr, indices, seeds, [8, 4, 2], 12345)
    for got, rb in zip(blocks.host(), ref):
        assert np.array_equal(got[0], rb.indptr) and np.array_equal(got[1], rb.gid)
        assert np.array_equal(got[2], rb.lid) and np.array_equal(got[3], rb.dst_lid)
        assert np.array_equal(got[4], rb.nodes)


@pytest.mark.parametrize("n_keep,n_add,bound", [(0, 0, 1), (1, 0, 5), (300, 2000, 5000),
                                                (5000, 200000, 233000), (7, 50000, 64)])
def test_unique_relabel_standalone(n_keep, n_add, bound):
    rng = np.random.default_rng(n_add)
    keep = rng.choice(bound, size=n_keep, replace=False).astype(np.int32)
    add = rng.integers(0, bound, size=n_add).astype(np.int32)
    dev = lambda a: torch.from_numpy(a).cuda() if a.size else torch.zeros(0, dtype=torch.int32, device="cuda")
    uniq = torch.full((n_keep + n_add + 1,), -7, dtype=torch.int32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int64, device="cuda")
    add_lid = torch.empty(max(n_add, 1), dtype=torch.int32, device="cuda")[:n_add]
    keep_lid = torch.empty(max(n_keep, 1), dtype=torch.int32, device="cuda")[:n_keep]
    ws = torch.empty(gm.gnn_relabel_workspace_size(bound), dtype=torch.uint8, device="cuda")
    gm.gnn_unique_relabel(dev(keep), dev(add), bound, uniq, nu, add_lid, keep_lid, ws)
    assert gm.gnn_read_device_status(ws) == gm.GNN_OK
    u, lid, dl = oracle.relabel(keep, add)
    assert nu.item() == len(u)
    assert np.array_equal(uniq[:len(u)].cpu().numpy(), u)
    assert np.array_equal(add_lid.cpu().numpy(), lid)
    assert np.array_equal(keep_lid.cpu().numpy(), dl)


def test_unique_relabel_device_count():
    add = torch.tensor([9, 3, 9, 1, 7, 7], dtype=torch.int32, device="cuda")
    keep = torch.tensor([4], dtype=torch.int32, device="cuda")
    n_add = torch.tensor([4], dtype=torch.int64, device="cuda")   # only the first 4 count
    uniq = torch.full((8,), -1, dtype=torch.int32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int64, device="cuda")
    add_lid = torch.full((6,), -1, dtype=torch.int32, device="cuda")
    keep_lid = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(gm.gnn_relabel_workspace_size(10), dtype=torch.uint8, device="cuda")
    gm.gnn_unique_relabel(keep, add, 10, uniq, nu, add_lid, keep_lid, ws, d_n_add=n_add)
    assert nu.item() == 4
    assert uniq[:4].tolist() == [1, 3, 4, 9]
    assert add_lid[:4].tolist() == [3, 1, 3, 0] and keep_lid.tolist() == [2]


@pytest.mark.parametrize("d,ld", [(602, 604), (13, 13), (64, 64), (100, 100), (128, 132), (3, 4)])
def test_gather_standalone(d, ld):
    rng = np.random.default_rng(d)
    n = 3000
    x = rng.standard_normal((n, d)).astype(np.float32)
    fs = _store(x, ld)
    ids = rng.integers(0, n, size=1777).astype(np.int32)
    out = torch.full((1777, ld + 4), 7.0, dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    gm.gnn_gather_features(fs, torch.from_numpy(ids).cuda(), out, d_status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    ref = oracle.gather(x, ids, d)
    assert np.array_equal(out[:, :d].cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert torch.all(out[:, d:] == 7.0)       # columns past d untouched


def test_gather_out_of_range_reported():
    x = np.ones((10, 4), np.float32)
    fs = _store(x, 4)
    out = torch.zeros(3, 4, dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    gm.gnn_gather_features(fs, torch.tensor([1, 10, -1], dtype=torch.int32, device="cuda"), out,
                           d_status=st)
    torch.cuda.synchronize()
    assert st.item() == gm.GNN_ERR_OUT_OF_RANGE


# row widths covering every lane layout of the mean: 16 / 32 lanes per row, 64 lanes with 1-4
# chunk groups per lane, several slabs per row (d > 1024), a ragged last chunk, a scalar path
@pytest.mark.parametrize("d,ld", [(602, 604), (7, 7), (128, 128), (13, 16), (100, 100), (130, 132),
                                  (300, 300), (700, 704), (1000, 1000), (1030, 1032), (2050, 2052)])
def test_mean_standalone(d, ld):
    rng = np.random.default_rng(d + 1)
    n_src, n_dst = 500, 300
    src = rng.uniform(-1, 1, size=(n_src, d)).astype(np.float32)
    counts = rng.integers(0, 26, size=n_dst)
    counts[:5] = 0
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    lid = rng.integers(0, n_src, size=int(counts.sum())).astype(np.int32)
    out = torch.zeros(n_dst, ld, dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    gm.gnn_mean_aggregate(torch.from_numpy(indptr).cuda(), torch.from_numpy(lid).cuda(),
                          device_table(src, ld), d, out, d_status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    ref = oracle.mean_aggregate(indptr, lid, src)
    err = np.abs(out[:, :d].cpu().numpy().astype(np.float64) - ref).max()
    assert err <= 1e-5 * np.abs(src).max()
    assert np.all(out[:5, :d].cpu().numpy() == 0)


def test_feature_cache_is_transparent(tiny):
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    table = device_table(x, 64)
    plain = gm.gnn_feature_store_create(table, 64)
    deg = np.diff(indptr)
    hot = np.argsort(-deg, kind="stable")[:3000].astype(np.int32)
    cached = gm.gnn_feature_store_create(table, 64, 3000, torch.from_numpy(hot).cuda())
    seeds = order[:cfg.batch]
    a, sa = run_minibatch(dg, plain, seeds, cfg.fanouts, 3)
    b, sb = run_minibatch(dg, cached, seeds, cfg.fanouts, 3)
    assert sa == sb == gm.GNN_OK
    nodes = b[0].blocks.host()[-1][4]
    nv = len(nodes)
    assert torch.equal(a[0].x[:nv], b[0].x[:nv]) and torch.equal(a[0].h[0], b[0].h[0])
    # the gather reports the rows it took from the cache
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty(len(nodes), 64, dtype=torch.float32, device="cuda")
    gm.gnn_gather_features(cached, torch.from_numpy(nodes).cuda(), out, d_hits=hits)
    assert hits.item() == len(np.intersect1d(nodes, hot))
    assert torch.equal(out, b[0].x[:len(nodes)])


def test_host_resident_table_zero_copy(tiny):
    cfg, indptr, indices, x, order = tiny
    host = torch.zeros(cfg.num_nodes, 64, dtype=torch.float32, pin_memory=True)
    host.copy_(torch.from_numpy(x))
    fs_host = gm.gnn_feature_store_create(host, 64)
    deg = np.diff(indptr)
    hot = np.argsort(-deg, kind="stable")[:1000].astype(np.int32)
    fs_mix = gm.gnn_feature_store_create(host, 64, 1000, torch.from_numpy(hot).cuda())
    dg = device_graph(indptr, indices)
    seeds = order[:cfg.batch]
    ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, 11)
    for fs in (fs_host, fs_mix):
        outs, st = run_minibatch(dg, fs, seeds, cfg.fanouts, 11)
        assert st == gm.GNN_OK
        compare_with_oracle(outs[0], ref, cfg.d)


@pytest.mark.parametrize("budget", [0, 3000, 40000, None])     # None: room for every row
@pytest.mark.parametrize("where", ["host", "hbm"])
def test_adjacency_host_resident_and_cached(tiny, where, budget):
    """Neighbour ids read from pinned host memory in place and/or from an HBM adjacency cache of
    several sizes: the same blocks, rows and means as the oracle (a super-batch of 8)."""
    from graph_mini_pipeline_amd.hotness import presample_adjacency_order
    cfg, indptr, indices, x, order = tiny
    base = device_graph(indptr, indices)
    if where == "host":
        ind = torch.empty(len(indices), dtype=torch.int32, pin_memory=True)
        ind.copy_(torch.from_numpy(indices))
    else:
        ind = base.indices
    bare = gm.DeviceGraph(base.num_nodes, base.indptr, ind)
    pre = torch.from_numpy(order[-4 * cfg.batch:].copy()).cuda()
    hot = presample_adjacency_order(base, base.indptr, pre, cfg.batch, cfg.fanouts, 99)
    assert torch.unique(hot).numel() == hot.numel() > 0
    cap = len(indices) if budget is None else budget
    cache = gm.gnn_adjacency_cache_create(bare, hot, cap)
    deg = np.diff(indptr)[hot.cpu().numpy()]
    assert cache.entries <= cap and cache.rows <= int((deg > 0).sum())
    if budget is None:
        assert cache.rows == int((deg > 0).sum()) and cache.entries == int(deg.sum())
    dg = gm.DeviceGraph(base.num_nodes, base.indptr, ind, adjacency=cache if cap else None)
    fs = _store(x)
    ptr = [j * cfg.batch for j in range(9)]
    seeds = order[:ptr[-1]]
    outs, st = run_minibatch(dg, fs, seeds, cfg.fanouts, 13, group_ptr=ptr)
    assert st == gm.GNN_OK
    for j in (0, 7):
        ref = oracle.minibatch(indptr, indices, x, seeds[ptr[j]:ptr[j + 1]], cfg.fanouts, 13)
        compare_with_oracle(outs[j], ref, cfg.d)


def test_repeat_runs_identical(tiny):
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    fs = _store(x)
    seeds = order[:cfg.batch]
    a, _ = run_minibatch(dg, fs, seeds, [15, 10, 5], 21)
    b, _ = run_minibatch(dg, fs, seeds, [15, 10, 5], 21)
    cnt = a[0].blocks.counts.cpu().tolist()
    rows = [len(seeds), cnt[1], cnt[3]]
    for l in range(3):
        assert torch.equal(a[0].h[l][:rows[l]], b[0].h[l][:rows[l]])
    assert torch.equal(a[0].x[:cnt[5]], b[0].x[:cnt[5]])
    for ha, hb in zip(a[0].blocks.host(), b[0].blocks.host()):
        for u, v in zip(ha, hb):
            assert np.array_equal(u, v)


SUPER_MODES = ["auto", "full", "compact"]


@pytest.mark.parametrize("mode", SUPER_MODES)
def test_superbatch_equals_separate_runs(tiny, mode):
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    fs = _store(x)
    seeds = order[:700]
    ptr = [0, 256, 256, 600, 700]
    outs, st = run_minibatch(dg, fs, seeds, cfg.fanouts, 77, group_ptr=ptr,
                             opts=gm.Options(superbatch=mode))
    assert st == gm.GNN_OK
    for g in range(4):
        ref = oracle.minibatch(indptr, indices, x, seeds[ptr[g]:ptr[g + 1]], cfg.fanouts, 77)
        compare_with_oracle(outs[g], ref, cfg.d)


@pytest.mark.parametrize("mode", SUPER_MODES)
def test_superbatch_of_16_with_overlap(tiny, mode):
    # 16 sub-batches; sub-batches may share seeds (each must be distinct within itself)
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    fs = _store(x)
    parts = [order[i * 40:(i + 1) * 40 + 13] for i in range(16)]   # consecutive parts overlap
    seeds = np.concatenate(parts)
    ptr = np.concatenate([[0], np.cumsum([len(p) for p in parts])]).tolist()
    outs, st = run_minibatch(dg, fs, seeds, [12, 6, 3], 5150, group_ptr=ptr,
                             opts=gm.Options(superbatch=mode))
    assert st == gm.GNN_OK
    for g in (0, 7, 15):
        ref = oracle.minibatch(indptr, indices, x, parts[g], [12, 6, 3], 5150)
        compare_with_oracle(outs[g], ref, cfg.d)


@pytest.mark.parametrize("mode", SUPER_MODES)
def test_superbatch_duplicate_within_sub_batch_reported(tiny, mode):
    cfg, indptr, indices, x, order = tiny
    seeds = np.array([1, 2, 3, 3, 4], np.int32)      # sub-batch 1 holds 3 twice
    _, st = run_minibatch(device_graph(indptr, indices), _store(x), seeds, [3], 1,
                          group_ptr=[0, 2, 5], opts=gm.Options(superbatch=mode))
    assert st == gm.GNN_ERR_INVALID_ARG


@pytest.mark.parametrize("mode", SUPER_MODES)
def test_superbatch_out_of_range_seed_reported(tiny, mode):
    cfg, indptr, indices, x, order = tiny
    seeds = np.array([1, 2, 3, cfg.num_nodes, 4], np.int32)
    _, st = run_minibatch(device_graph(indptr, indices), _store(x), seeds, [3, 2], 1,
                          group_ptr=[0, 2, 5], opts=gm.Options(superbatch=mode))
    assert st == gm.GNN_ERR_OUT_OF_RANGE


@pytest.mark.parametrize("mode", ["full", "compact"])
def test_superbatch_single_node_graph_regions(mode):
    # two sub-batches on a star: every leaf's only neighbour is the hub, the hub has them all;
    # the union at hop 2 is the whole graph in both sub-batches
    indptr, indices = H.star(3000)
    x = np.random.default_rng(3).standard_normal((3001, 8)).astype(np.float32)
    seeds = np.array([5, 17, 2999, 0, 17, 40], np.int32)
    outs, st = run_minibatch(device_graph(indptr, indices), _store(x), seeds, [4, 3], 99,
                             group_ptr=[0, 3, 6], opts=gm.Options(superbatch=mode))
    assert st == gm.GNN_OK
    for g, (a, b) in enumerate([(0, 3), (3, 6)]):
        ref = oracle.minibatch(indptr, indices, x, seeds[a:b], [4, 3], 99)
        compare_with_oracle(outs[g], ref, 8)


@pytest.mark.parametrize("fanouts", [[10, 5], [25, 10], [3, 3, 3]])
def test_high_word_ranking_equals_exact_ranking(tiny, fanouts):
    # the sampler's default selection (ranks by the keys' high words, full order on a tie at the
    # fanout-th place) against ranking every node by (key, position); both against the oracle
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    fs = _store(x)
    seeds = order[:512]
    fast, st = run_minibatch(dg, fs, seeds, fanouts, 31337)
    assert st == gm.GNN_OK
    exact, st = run_minibatch(dg, fs, seeds, fanouts, 31337, opts=gm.Options(exact_rank=True))
    assert st == gm.GNN_OK
    for hf, he in zip(fast[0].blocks.host(), exact[0].blocks.host()):
        for u, v in zip(hf, he):
            assert np.array_equal(u, v)
    compare_with_oracle(fast[0], oracle.minibatch(indptr, indices, x, seeds, fanouts, 31337), cfg.d)


def test_superbatch_compact_seeds_beyond_the_id_range():
    # G times the per-sub-batch seed count exceeds the number of nodes, so the first union level
    # is the sorted union of the seeds rather than their concatenation; sub-batches overlap
    indptr, indices = H.random_csr(300, 6.0, 41)
    x = np.random.default_rng(41).standard_normal((300, 16)).astype(np.float32)
    perm = np.random.default_rng(42).permutation(300).astype(np.int32)
    parts = [perm[i * 60:i * 60 + 110] for i in range(4)]     # 4 x 110 > 300 ids
    seeds = np.concatenate(parts)
    ptr = np.concatenate([[0], np.cumsum([len(p) for p in parts])]).tolist()
    outs, st = run_minibatch(device_graph(indptr, indices), _store(x), seeds, [5, 3], 4242,
                             group_ptr=ptr, opts=gm.Options(superbatch="compact"))
    assert st == gm.GNN_OK
    for g in range(4):
        ref = oracle.minibatch(indptr, indices, x, parts[g], [5, 3], 4242)
        compare_with_oracle(outs[g], ref, 16)


class _BothModes(gm.Options):
    def c(self):
        o = super().c()
        o.flags |= gm.GNN_SUPERBATCH_FULL | gm.GNN_SUPERBATCH_COMPACT
        return o


def test_superbatch_both_flags_rejected(tiny):
    cfg, indptr, indices, x, order = tiny
    with pytest.raises(ValueError):
        gm.Options(superbatch="both").c()
    with pytest.raises(gm.GnnError) as e:
        run_minibatch(device_graph(indptr, indices), _store(x), order[:20], [3], 1,
                      group_ptr=[0, 10, 20], opts=_BothModes())
    assert e.value.status == gm.GNN_ERR_INVALID_ARG


def test_superbatch_too_large_rejected(tiny):
    cfg, indptr, indices, x, order = tiny
    with pytest.raises(gm.GnnError) as e:
        run_minibatch(device_graph(indptr, indices), _store(x), order[:17], [3], 1,
                      group_ptr=list(range(18)))
    assert e.value.status == gm.GNN_ERR_UNSUPPORTED


# Giant rows: two hubs of 10^6 and 4*10^4 in-neighbours in one frontier, with fanouts on either
# side of the largest that the 16-lane (26) and one-wavefront (104) classes take, and the largest
# fanout the library supports (832: a quarter of a workgroup's candidate capacity).
def _two_hubs(D1=1_000_000, D2=40_000):
    rows = [list(range(2, 2 + D1)), list(range(3, 3 + D2))] + [[0, 1] for _ in range(D1 + 1)]
    return H.csr_from_rows(rows)


@pytest.mark.parametrize("fanouts", [[5, 3], [26, 2], [27, 2], [104, 1], [105, 1], [200, 1], [832, 1]])
def test_giant_rows(fanouts):
    indptr, indices = _two_hubs()
    N = len(indptr) - 1
    x = np.random.default_rng(11).standard_normal((N, 8)).astype(np.float32)
    seeds = np.array([0, 1, 7, 50_000], np.int32)
    outs, st = run_minibatch(device_graph(indptr, indices), _store(x), seeds, fanouts, 4242)
    assert st == gm.GNN_OK
    ref = oracle.minibatch(indptr, indices, x, seeds, fanouts, 4242)
    compare_with_oracle(outs[0], ref, 8)


GATHER_MODES = {"auto": gm.Options(), "interleaved": gm.Options(gather="interleaved"),
                "batched": gm.Options(gather="batched")}


def _stores(x, ld, hot_rows, indptr):
    """The four kinds of feature store over the same rows: HBM, HBM + cache, host, host + cache."""
    n, d = x.shape
    dev = device_table(x, ld)
    host = torch.zeros(n, ld, dtype=torch.float32, pin_memory=True)
    host[:, :d].copy_(torch.from_numpy(x))
    hot = torch.from_numpy(np.argsort(-np.diff(indptr), kind="stable")[:hot_rows].astype(np.int32)).cuda()
    return {"hbm": gm.gnn_feature_store_create(dev, d),
            "hbm_cache": gm.gnn_feature_store_create(dev, d, hot_rows, hot),
            "host": gm.gnn_feature_store_create(host, d),
            "host_cache": gm.gnn_feature_store_create(host, d, hot_rows, hot)}


@pytest.mark.parametrize("mode", sorted(GATHER_MODES))
@pytest.mark.parametrize("store", ["hbm", "hbm_cache", "host", "host_cache"])
def test_gather_modes_match_oracle(tiny, mode, store):
    # a super-batch with an empty sub-batch, through each feature-store kind and gather layout
    cfg, indptr, indices, x, order = tiny
    fs = _stores(x, 64, 1500, indptr)[store]
    seeds = order[:700]
    ptr = [0, 256, 256, 600, 700]
    outs, st = run_minibatch(device_graph(indptr, indices), fs, seeds, cfg.fanouts, 404,
                             group_ptr=ptr, opts=GATHER_MODES[mode])
    assert st == gm.GNN_OK
    for g in range(4):
        ref = oracle.minibatch(indptr, indices, x, seeds[ptr[g]:ptr[g + 1]], cfg.fanouts, 404)
        compare_with_oracle(outs[g], ref, cfg.d)


@pytest.mark.parametrize("d,ld", [(5, 5), (100, 100), (602, 604)])
@pytest.mark.parametrize("store", ["hbm", "host_cache"])
def test_batched_gather_row_widths(tiny, d, ld, store):
    # unaligned rows (5 floats) take the flat kernel; 100 and 602 floats the 32- and 64-lane groups
    cfg, indptr, indices, _, order = tiny
    x = np.random.default_rng(d).standard_normal((cfg.num_nodes, d)).astype(np.float32)
    fs = _stores(x, ld, 2000, indptr)[store]
    seeds = order[:600]
    ptr = [0, 100, 350, 600]
    outs, st = run_minibatch(device_graph(indptr, indices), fs, seeds, [6, 4], 31, group_ptr=ptr,
                             opts=gm.Options(gather="batched"))
    assert st == gm.GNN_OK
    for g in range(3):
        ref = oracle.minibatch(indptr, indices, x, seeds[ptr[g]:ptr[g + 1]], [6, 4], 31)
        compare_with_oracle(outs[g], ref, d)


@pytest.mark.parametrize("mode", ["full", "compact"])
@pytest.mark.parametrize("d,ld", [(150, 152), (602, 604), (150, 151)])
def test_union_gather(tiny, mode, d, ld):
    """Rows wider than 128 floats from a table in HBM: a super-batch gathers the union of its
    sub-batches' node sets once and stores each row to every sub-batch's X that holds it (rows
    that are not 16-byte aligned, ld = 151, gather per sub-batch).  Overlapping and empty
    sub-batches, both relabel modes."""
    cfg, indptr, indices, _, order = tiny
    x = np.random.default_rng(d + ld).standard_normal((cfg.num_nodes, d)).astype(np.float32)
    fs = gm.gnn_feature_store_create(device_table(x, ld), d)
    seeds = np.concatenate([order[:300], order[150:420], order[:0], order[400:460], order[0:50]])
    ptr = [0, 300, 570, 570, 630, 680]
    outs, st = run_minibatch(device_graph(indptr, indices), fs, seeds, [7, 5], 57, group_ptr=ptr,
                             opts=gm.Options(superbatch=mode))
    assert st == gm.GNN_OK
    for g in range(5):
        ref = oracle.minibatch(indptr, indices, x, seeds[ptr[g]:ptr[g + 1]], [7, 5], 57)
        compare_with_oracle(outs[g], ref, d)


class _BothGather(gm.Options):
    def c(self):
        o = super().c()
        o.flags |= gm.GNN_GATHER_INTERLEAVED | gm.GNN_GATHER_BATCHED
        return o


def test_gather_both_flags_rejected(tiny):
    cfg, indptr, indices, x, order = tiny
    with pytest.raises(ValueError):
        gm.Options(gather="both").c()
    with pytest.raises(gm.GnnError) as e:
        run_minibatch(device_graph(indptr, indices), _store(x), order[:20], [3], 1,
                      group_ptr=[0, 10, 20], opts=_BothGather())
    assert e.value.status == gm.GNN_ERR_INVALID_ARG


@pytest.mark.parametrize("mode", SUPER_MODES)
@pytest.mark.parametrize("fanouts", [[7], [12, 6], [12, 6, 3]])
@pytest.mark.parametrize("ld", [64, 66])
def test_shared_outer_means(tiny, mode, fanouts, ld):
    # batched gathers from a table in HBM: the outermost means are taken once per node of the union
    # frontier and stored to every sub-batch that holds the node; sub-batches overlap, one is
    # empty; rows 16-byte aligned (64 floats) or not (66: the flat kernels)
    cfg, indptr, indices, x, order = tiny
    dg = device_graph(indptr, indices)
    fs = _store(x, ld)
    parts = [order[i * 50:(i + 1) * 50 + 20] for i in range(6)] + [order[:0]] + [order[100:180]]
    seeds = np.concatenate(parts)
    ptr = np.concatenate([[0], np.cumsum([len(p) for p in parts])]).tolist()
    outs, st = run_minibatch(dg, fs, seeds, fanouts, 808, group_ptr=ptr,
                             opts=gm.Options(superbatch=mode, gather="batched"))
    assert st == gm.GNN_OK
    for g in range(len(parts)):
        ref = oracle.minibatch(indptr, indices, x, parts[g], fanouts, 808)
        compare_with_oracle(outs[g], ref, cfg.d)


# Lists far shorter than the id range are relabelled by one workgroup that sorts them in LDS
# instead of through a bitmap over every id: over 2^30 ids every one of these cases takes that path
# (the last one with its largest list), and must equal the oracle like every other relabel.
@pytest.mark.parametrize("n_keep,n_add,bound,distinct",
                         [(0, 0, 1 << 30, None), (1, 0, 1 << 30, None), (300, 2000, 1 << 30, None),
                          (700, 7000, 1 << 30, 50), (2000, 6000, 1 << 30, None),
                          (5000, 11384, 1 << 30, None)])
def test_unique_relabel_short_lists(n_keep, n_add, bound, distinct):
    rng = np.random.default_rng(n_add + 17)
    keep = rng.choice(bound, size=n_keep, replace=False).astype(np.int32) if n_keep else np.zeros(0, np.int32)
    if distinct:   # many repeats of few ids (a hub sampled by many destinations)
        pool = rng.choice(bound, size=distinct, replace=False)
        add = rng.choice(pool, size=n_add).astype(np.int32)
    else:
        add = rng.integers(0, bound, size=n_add).astype(np.int32)
    dev = lambda a: torch.from_numpy(a).cuda() if a.size else torch.zeros(0, dtype=torch.int32, device="cuda")
    uniq = torch.full((n_keep + n_add + 1,), -7, dtype=torch.int32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int64, device="cuda")
    add_lid = torch.empty(max(n_add, 1), dtype=torch.int32, device="cuda")[:n_add]
    keep_lid = torch.empty(max(n_keep, 1), dtype=torch.int32, device="cuda")[:n_keep]
    ws = torch.empty(gm.gnn_relabel_workspace_size(bound), dtype=torch.uint8, device="cuda")
    gm.gnn_unique_relabel(dev(keep), dev(add), bound, uniq, nu, add_lid, keep_lid, ws)
    assert gm.gnn_read_device_status(ws) == gm.GNN_OK
    u, lid, dl = oracle.relabel(keep, add)
    assert nu.item() == len(u)
    assert np.array_equal(uniq[:len(u)].cpu().numpy(), u)
    assert np.array_equal(add_lid.cpu().numpy(), lid)
    assert np.array_equal(keep_lid.cpu().numpy(), dl)


@pytest.fixture(scope="module")
def sparse_wide():
    """2M nodes, few edges (degrees 0..7, repeats and self-loops allowed): batches of a few dozen
    seeds have lists far shorter than the id range."""
    rng = np.random.default_rng(2024)
    n = 2_000_000
    deg = rng.integers(0, 8, size=n)
    indptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    indices = rng.integers(0, n, size=int(indptr[-1])).astype(np.int32)
    x = rng.standard_normal((n, 8)).astype(np.float32)
    return indptr, indices, x


@pytest.mark.parametrize("relabel", ["sort", "bitmap"])
@pytest.mark.parametrize("mode", [None, "compact"])
def test_short_list_relabel_in_minibatch(sparse_wide, mode, relabel):
    """gnn_minibatch on the wide sparse graph with either relabel path forced: one batch (every
    hop's relabel sorts, or none does), and a super-batch of three overlapping sub-batches
    relabelled in the union's positions (the seeds' union sorts and leaves its bits in the
    node-id bitmap for the later hops)."""
    indptr, indices, x = sparse_wide
    dg = device_graph(indptr, indices)
    fs = _store(x)
    rng = np.random.default_rng(5)
    seeds = rng.choice(len(indptr) - 1, size=96, replace=False).astype(np.int32)
    fanouts = [4, 3]
    seed64 = gm.gnn_batch_seed(11, 3)
    if mode is None:
        outs, st = run_minibatch(dg, fs, seeds[:64], fanouts, seed64, gm.Options(relabel=relabel))
        parts = [seeds[:64]]
    else:
        sb = np.concatenate([seeds[:40], seeds[20:70], seeds[60:96]])
        ptr = [0, 40, 90, 126]
        outs, st = run_minibatch(dg, fs, sb, fanouts, seed64,
                                 gm.Options(superbatch=mode, relabel=relabel), group_ptr=ptr)
        parts = [sb[ptr[g]:ptr[g + 1]] for g in range(3)]
    assert st == gm.GNN_OK
    for out, sd in zip(outs, parts):
        ref = oracle.minibatch(indptr, indices, x, sd, fanouts, seed64)
        compare_with_oracle(out, ref, x.shape[1])


def test_short_list_relabel_reports_bad_seeds(sparse_wide):
    indptr, indices, x = sparse_wide
    dg = device_graph(indptr, indices)
    fs = _store(x)
    sort = gm.Options(relabel="sort")
    seeds = np.array([5, 77, 123456, 77, 9], dtype=np.int32)        # 77 twice
    _, st = run_minibatch(dg, fs, seeds, [3, 2], gm.gnn_batch_seed(0, 0), sort)
    assert st == gm.GNN_ERR_INVALID_ARG
    seeds = np.array([5, 77, len(indptr) - 1, 9], dtype=np.int32)   # one past the last node
    _, st = run_minibatch(dg, fs, seeds, [3, 2], gm.gnn_batch_seed(0, 0), sort)
    assert st == gm.GNN_ERR_OUT_OF_RANGE


_FAULT_CHILD = r'''
import sys
sys.path.insert(0, %r)
import numpy as np, torch
import graph_mini_pipeline_amd as gm, synth
from tests.gpu_util import device_graph, device_table, run_minibatch
cfg = synth.CONFIGS["tiny"]
g = synth.build_graph(cfg)
x = torch.empty(cfg.num_nodes, cfg.d, dtype=torch.float32)
synth.make_features(cfg, x)
dg = device_graph(g.indptr.numpy(), g.indices.numpy())
fs = gm.gnn_feature_store_create(device_table(x.numpy(), cfg.d), cfg.d)
seeds = synth.epoch_seed_order(cfg).numpy()[:64]
try:
    _, st = run_minibatch(dg, fs, seeds, cfg.fanouts, gm.gnn_batch_seed(0, 0))
    print("status", st)
except gm.GnnError as e:
    print("raised", e.status)
'''


@pytest.mark.parametrize("fault,want", [(None, "status 0"), ("launch", "raised %d" % gm.GNN_ERR_HIP)])
def test_fault_injection_in_a_child_process(fault, want):
    """GNN_FAULT=launch makes a mini-batch that otherwise succeeds fail with GNN_ERR_HIP before any
    work is enqueued (the child process reads the variable; this process is not affected)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ)
    env.pop("GNN_FAULT", None)
    if fault:
        env["GNN_FAULT"] = fault
    r = subprocess.run([sys.executable, "-c", _FAULT_CHILD % root], env=env, capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == want
