"""Parity on the billion-edge workload: 250M nodes, 4B edges (int64 indptr), 64-d features in
pinned host memory (64 GB) with a 16 GiB HBM hot-row cache (26.8% of the rows) ranked by
pre-sampling, batches of 4096 seeds, fanouts [15, 10, 5], super-batches of 8 and of 16 (the benchmark's).  Two sub-batches of
each are compared with the oracle
(bit-exact blocks and gathered rows, means within 1e-5 * max|X|); the gather must hit the cache
for some rows and read the rest from host memory.  With the Dynamic-Cache on (GARDEN Sec. IV.B,
eq. 5-6) at this size, properties that hold at any size are checked: gathered rows equal the
table's, cache hits equal the rows held by the static cache or by resident members, and each
refresh's members are a top K_dyn of its own scores."""
import pytest
import torch

import oracle
import synth
from tests.gpu_util import compare_with_oracle

pytestmark = pytest.mark.gpu

gm = pytest.importorskip("graph_mini_pipeline_amd")


@pytest.fixture(scope="module")
def billion():
    from graph_mini_pipeline_amd.hotness import presample_hot_order
    cfg = synth.CONFIGS["billion"]
    dev = torch.device("cuda")
    g = synth.build_graph(cfg, device=dev)
    table = torch.empty(cfg.num_nodes, cfg.ld, dtype=torch.float32, pin_memory=True)
    synth.make_features(cfg, table, device=dev)
    order = synth.epoch_seed_order(cfg, 0, device=dev).contiguous()
    dg = gm.DeviceGraph(cfg.num_nodes, g.indptr, g.indices)
    rows = cfg.cache_bytes // (cfg.ld * 4)
    pre = synth.presample_seeds(cfg, 64, device=dev)
    hot = presample_hot_order(dg, g.indptr, pre, cfg.batch, cfg.fanouts,
                              synth.sub_seed(cfg.rng_seed, 6), rows)
    fs = gm.gnn_feature_store_create(table, cfg.d, rows, hot)
    fs.hot_order = hot   # the static cache's rows, for the Dynamic-Cache test's own store
    host = (g.indptr.cpu().numpy(), g.indices.cpu().numpy(), table.numpy(), order.cpu().numpy())
    yield cfg, dg, fs, order, host
    del fs, dg, g, table, host
    torch.cuda.empty_cache()
    if hasattr(torch._C, "_host_emptyCache"):   # hand the pinned table back to the system
        torch._C._host_emptyCache()


@pytest.mark.parametrize("G,check", [(8, (0, 5)), (16, (9, 15))])
def test_billion_superbatch(billion, G, check):
    cfg, dg, fs, order, (indptr, indices, x, order_h) = billion
    seed64 = gm.gnn_batch_seed(cfg.rng_seed, 0)
    ptr = [j * cfg.batch for j in range(G + 1)]
    outs = [gm.MinibatchOut(gm.gnn_capacity(cfg.batch, cfg.fanouts, cfg.num_nodes), cfg.d, cfg.ld)
            for _ in range(G)]
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, cfg.num_nodes)
    ws = torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes, G), dtype=torch.uint8, device="cuda")
    gm.gnn_minibatch(dg, fs, order[:G * cfg.batch], ptr, cfg.fanouts, seed64, outs, ws)
    assert gm.gnn_read_device_status(ws) == gm.GNN_OK
    K = len(cfg.fanouts)
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    gm.gnn_gather_features(fs, outs[0].blocks.nodes[K - 1], outs[0].x,
                           d_n=outs[0].blocks.counts[2 * K - 1:2 * K], d_hits=hits)
    nv = int(outs[0].blocks.counts[2 * K - 1].item())
    assert 0 < int(hits.item()) < nv, (int(hits.item()), nv)
    for j in check:
        seeds = order_h[j * cfg.batch:(j + 1) * cfg.batch]
        ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
        compare_with_oracle(outs[j], ref, cfg.d)


def test_billion_dynamic_cache(billion):
    """Four super-batches of 16 through a store with the Dynamic-Cache (refreshed after each)."""
    import numpy as np
    cfg, dg, fs0, order, _ = billion
    hot = fs0.hot_order
    rows = hot.numel()
    N, K = cfg.num_nodes, len(cfg.fanouts)
    fs = gm.gnn_feature_store_create(fs0.table, cfg.d, rows, hot)
    k_dyn = 1 << 20
    gm.gnn_feature_store_enable_dynamic(fs, 0.995, k_dyn, 16, auto=True)
    static = torch.zeros(N, dtype=torch.bool, device="cuda")
    static[hot.long()] = True
    G = 16
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, N)
    ws = torch.empty(gm.gnn_workspace_size(caps, N, G), dtype=torch.uint8, device="cuda")
    outs = [gm.MinibatchOut(caps, cfg.d, cfg.ld) for _ in range(G)]
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    score = torch.empty(N, dtype=torch.float64, device="cuda")
    member = torch.zeros(N, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(4)
    table = fs0.table
    for step in range(4):
        sb = 40 + step                       # super-batches the other tests do not use
        seeds = order[sb * G * cfg.batch:(sb + 1) * G * cfg.batch]
        held = static | (member == 1)        # resident before this call's gathers
        hits.zero_()
        gm.gnn_minibatch(dg, fs, seeds, [j * cfg.batch for j in range(G + 1)], cfg.fanouts,
                         gm.gnn_batch_seed(cfg.rng_seed, sb), outs, ws, gm.Options(d_hits=hits))
        assert gm.gnn_read_device_status(ws) == gm.GNN_OK
        want = 0
        checked = set(rng.choice(G, 3, replace=False).tolist())
        for j, out in enumerate(outs):
            nv = int(out.blocks.counts[2 * K - 1].item())
            vk = out.blocks.nodes[K - 1][:nv].long()
            want += int(held[vk].sum().item())
            if j in checked:   # rows of three sub-batches against the table
                idx = vk.cpu()
                assert torch.equal(out.x[:nv, :cfg.d].cpu().view(torch.int32),
                                   table[idx][:, :cfg.d].view(torch.int32)), (step, j)
        assert int(hits.item()) == want, (step, int(hits.item()), want)
        gm.gnn_dyn_cache_state(fs, score, member)
        torch.cuda.synchronize()
        info = gm.gnn_dyn_cache_query(fs)
        assert info["refreshes"] == step + 1 and info["steps"] == (step + 1) * G
        mem = member > 0
        assert int(mem.sum().item()) == info["members"] <= k_dyn
        assert not bool((mem & static).any().item())
        # the members are a top K_dyn of the scores the refresh saw (the scores read now)
        pos = (score > 0) & ~static
        m = min(k_dyn, int(pos.sum().item()))
        assert info["members"] == m
        tau = torch.topk(score[pos], m).values[-1]
        assert bool((score[mem] >= tau * (1 - 1e-12)).all().item())
        assert int(((score > tau * (1 + 1e-12)) & pos & ~mem).sum().item()) == 0
        assert info["resident"] == int((member == 1).sum().item())
    fs.close()
