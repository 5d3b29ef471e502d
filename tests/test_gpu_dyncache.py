"""The Dynamic-Cache (GARDEN Sec. IV.B, eq. (5)-(6)) through the C ABI against the oracle's policy.

Scores: relative error <= 1e-10 (the device keeps w_t * Score(v, t) with w_t = gamma^-t and adds
each mini-batch's weight with fp64 atomics; the oracle decays every score in every step; both are
fp64, so they differ by rounding only).  Members: a refresh's members are a valid top K_dyn of the
oracle's scores at that refresh -- every node scored clearly above the K-th largest score is a
member, every member is scored no lower than it (up to the same relative 1e-10), and the count is
min(K_dyn, nodes with a positive score) -- since near-equal scores may round either way.  Gathered
rows: bit-exact with the table whatever the cache holds, and the cache-hit count equals the rows
held by the static cache or by the resident members at the time of the gather.  Residency: a
refresh reserves rows for the nodes it takes in and copies nothing; a member's row becomes
resident at the first refresh (or, frozen, publish) after a gather read it while it was a member,
and stays so while it remains a member (Residency below).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import compare_with_oracle, device_graph, device_table, run_minibatch

pytestmark = pytest.mark.gpu

gm = pytest.importorskip("graph_mini_pipeline_amd")

RTOL = 1e-10


def check_members(members, score, is_static, k):
    """members: ids holding a Dynamic-Cache row; score: the oracle's scores at the refresh."""
    members = np.asarray(members)
    pos = (score > 0) & (is_static == 0)
    m = min(k, int(pos.sum()))
    assert len(members) == m, f"{len(members)} members, expected {m}"
    if m == 0:
        return
    assert pos[members].all(), "a member without a positive score, or in the static cache"
    tau = np.sort(score[pos])[::-1][m - 1]
    assert (score[members] >= tau * (1 - RTOL)).all(), "a member ranked below the K-th score"
    above = np.nonzero(pos & (score > tau * (1 + RTOL)))[0]
    missing = np.setdiff1d(above, members)
    assert missing.size == 0, f"{missing.size} nodes ranked above the K-th score left out"


class Residency:
    """Expected resident members: the rows of the members requested since the last refresh become
    resident at the next one (before its new membership), and residents stay while members."""

    def __init__(self):
        self.members, self.resident, self.requested = set(), set(), set()

    def gathered(self, ids):
        self.requested |= set(np.asarray(ids).tolist()) & self.members

    def refreshed(self, new_members):
        filled = self.resident | (self.members & self.requested)
        self.members = set(np.asarray(new_members).tolist())
        self.resident = filled & self.members
        self.requested = set()


def skewed_ids(rng, n_nodes, n, perm):
    """Requested rows of one mini-batch: Zipf-like ranks (with repeats) mapped through a fixed
    permutation, so some nodes recur across mini-batches and within one."""
    r = (rng.zipf(1.25, size=n) - 1) % n_nodes
    return perm[r].astype(np.int32)


def device_state(fs, n):
    score = torch.empty(n, dtype=torch.float64, device="cuda")
    member = torch.empty(n, dtype=torch.uint8, device="cuda")
    gm.gnn_dyn_cache_state(fs, score, member)
    torch.cuda.synchronize()
    m = member.cpu().numpy()
    return score.cpu().numpy(), np.nonzero(m)[0], np.nonzero(m == 1)[0]


@pytest.mark.parametrize("d,ld", [(16, 16), (13, 13), (200, 200)],
                         ids=["rows16", "flat", "rows64"])
@pytest.mark.parametrize("auto", [False, True], ids=["update", "auto"])
def test_gather_observations_and_refreshes_match_the_oracle(d, ld, auto):
    rng = np.random.default_rng(11 + d)
    N, static_rows, K, T, gamma = 6000, 400, 250, 3, 0.8
    x = rng.standard_normal((N, d)).astype(np.float32)
    table = device_table(x, ld)
    perm = rng.permutation(N)
    # the static cache: 50 of the hottest nodes and a spread of colder ones, so hot residual rows
    # remain for the Dynamic-Cache
    hot = np.concatenate([perm[:50], perm[200::13][:static_rows - 50]]).astype(np.int32)
    assert np.unique(hot).size == static_rows
    fs = gm.gnn_feature_store_create(table, d, static_rows, torch.from_numpy(hot).cuda())
    gm.gnn_feature_store_enable_dynamic(fs, gamma, K, T, auto=auto)
    ref = oracle.DynCache(N, hot, gamma, K, T)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    members = resident = np.zeros(0, dtype=np.int64)
    res = Residency()
    refreshes = 0
    for step in range(16):
        ids = skewed_ids(rng, N, 700 + 37 * step, perm)
        held = np.union1d(hot, resident)
        hits.zero_()
        out = torch.full((ids.size, ld), float("nan"), dtype=torch.float32, device="cuda")
        gm.gnn_gather_features(fs, torch.from_numpy(ids).cuda(), out, d_hits=hits, d_status=status)
        ref.observe(ids)
        res.gathered(ids)
        if auto:
            did = ref.update()
        else:
            did = gm.gnn_dyn_cache_update(fs, d_status=status)
            assert did == ref.update()
        refreshes += did
        torch.cuda.synchronize()
        assert int(status.item()) == gm.GNN_OK
        got = out[:, :d].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), x[ids].view(np.uint32)), "gathered rows"
        assert int(hits.item()) == int(np.isin(ids, held).sum()), "cache hits"
        score, members, resident = device_state(fs, N)
        np.testing.assert_allclose(score, ref.score, rtol=RTOL, atol=0)
        if did:
            check_members(members, ref.score, ref.is_static, K)
            snap = ref.score.copy()
            res.refreshed(members)
        elif refreshes:
            check_members(members, snap, ref.is_static, K)
        else:
            assert members.size == 0
        assert set(members.tolist()) == res.members and set(resident.tolist()) == res.resident
        info = gm.gnn_dyn_cache_query(fs)
        assert info["steps"] == ref.steps and info["refreshes"] == ref.refreshes == refreshes
        assert info["members"] == members.size and info["resident"] == resident.size
    assert refreshes == 16 // T
    assert 0 < len(res.resident) < len(res.members)
    fs.close()


def test_refreshes_stop_after_max_refreshes():
    rng = np.random.default_rng(5)
    N, d = 3000, 8
    x = rng.standard_normal((N, d)).astype(np.float32)
    fs = gm.gnn_feature_store_create(device_table(x, d), d)
    gm.gnn_feature_store_enable_dynamic(fs, 0.9, 100, 2, max_refreshes=2)
    ref = oracle.DynCache(N, [], 0.9, 100, 2, max_refreshes=2)
    res = Residency()
    perm = rng.permutation(N)
    since = 0
    for step in range(9):
        ids = skewed_ids(rng, N, 500, perm)
        out = torch.empty(ids.size, d, dtype=torch.float32, device="cuda")
        gm.gnn_gather_features(fs, torch.from_numpy(ids).cuda(), out)
        ref.observe(ids)
        res.gathered(ids)
        since += 1
        frozen = ref.frozen
        did = gm.gnn_dyn_cache_update(fs)
        assert did == ref.update()
        assert np.array_equal(out.cpu().numpy(), x[ids])
        if did or (frozen and since >= 2):   # a refresh, or (frozen) a publish
            since = 0
            _, members, _ = device_state(fs, N)
            res.refreshed(members)
        _, members, resident = device_state(fs, N)
        assert set(resident.tolist()) == res.resident
    score, members, resident = device_state(fs, N)
    info = gm.gnn_dyn_cache_query(fs)
    assert info["frozen"] == 1 and info["refreshes"] == 2 and info["steps"] == 9
    np.testing.assert_allclose(score, ref.score, rtol=RTOL, atol=0)
    check_members(members, ref.score, ref.is_static, 100)
    assert info["resident"] == resident.size > 0
    fs.close()


def test_scores_stay_exact_across_the_weight_rescale():
    """gamma = 0.01: the weights w_t = 100^t pass 2^512 after 78 mini-batches and the scaled
    scores are brought back by 2^-512 at a refresh."""
    rng = np.random.default_rng(9)
    N, d, K, T, gamma = 2000, 4, 40, 10, 0.01
    x = rng.standard_normal((N, d)).astype(np.float32)
    fs = gm.gnn_feature_store_create(device_table(x, d), d)
    gm.gnn_feature_store_enable_dynamic(fs, gamma, K, T)
    ref = oracle.DynCache(N, [], gamma, K, T)
    perm = rng.permutation(N)
    for step in range(120):
        ids = skewed_ids(rng, N, 60, perm)
        out = torch.empty(ids.size, d, dtype=torch.float32, device="cuda")
        gm.gnn_gather_features(fs, torch.from_numpy(ids).cuda(), out)
        ref.observe(ids)
        did = gm.gnn_dyn_cache_update(fs)
        assert did == ref.update()
        if did:
            score, members, _ = device_state(fs, N)
            live = ref.score > 1e-250          # far below any member's score
            np.testing.assert_allclose(score[live], ref.score[live], rtol=1e-9, atol=0)
            check_members(members, ref.score, ref.is_static, K)
    fs.close()


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    g = synth.build_graph(cfg)
    x = torch.empty(cfg.num_nodes, cfg.d, dtype=torch.float32)
    synth.make_features(cfg, x)
    order = synth.epoch_seed_order(cfg)
    return cfg, g.indptr.numpy(), g.indices.numpy(), x.numpy(), order.numpy()


@pytest.mark.parametrize("interleaved", [False, True], ids=["batched", "interleaved"])
def test_superbatches_observe_each_sub_batch(tiny, interleaved):
    """gnn_minibatch with G = 4: each sub-batch's gather of V_K is one mini-batch, in sub-batch
    order; GNN_DYN_AUTO refreshes at the end of the call that completes an interval.  Every
    sub-batch's blocks, X and means equal the oracle's separate run."""
    cfg, indptr, indices, x, order = tiny
    N, d, G, batch = cfg.num_nodes, cfg.d, 4, 256
    deg = np.diff(indptr)
    hot = np.argsort(-deg, kind="stable")[:800].astype(np.int32)
    dg = device_graph(indptr, indices)
    fs = gm.gnn_feature_store_create(device_table(x, cfg.ld), d, hot.size,
                                     torch.from_numpy(hot).cuda())
    K, T, gamma = 500, 6, 0.9
    gm.gnn_feature_store_enable_dynamic(fs, gamma, K, T, auto=True)
    ref = oracle.DynCache(N, hot, gamma, K, T)
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    opts = gm.Options(gather="interleaved" if interleaved else "auto", d_hits=hits)
    snap = None
    resident = np.zeros(0, dtype=np.int64)
    res = Residency()
    for call in range(7):
        held = np.union1d(hot, resident)
        hits.zero_()
        lo = call * G * batch
        seeds = order[lo:lo + G * batch]
        ptr = [min(g * batch, seeds.size) for g in range(G + 1)]
        seed64 = gm.gnn_batch_seed(cfg.rng_seed, call)
        outs, st = run_minibatch(dg, fs, seeds, cfg.fanouts, seed64, opts=opts, group_ptr=ptr)
        assert st == gm.GNN_OK
        refs = oracle.superbatch(indptr, indices, x, seeds, ptr, cfg.fanouts, seed64)
        for g in range(G):
            compare_with_oracle(outs[g], refs[g], d)
            ref.observe(refs[g].blocks[-1].nodes)
            res.gathered(refs[g].blocks[-1].nodes)
        want = sum(int(np.isin(r.blocks[-1].nodes, held).sum()) for r in refs)
        assert int(hits.item()) == want, "cache hits"
        did = ref.update()
        score, members, resident = device_state(fs, N)
        if did:
            snap = ref.score.copy()
            res.refreshed(members)
        np.testing.assert_allclose(score, ref.score, rtol=RTOL, atol=0)
        if snap is not None:
            check_members(members, snap, ref.is_static, K)
        assert set(resident.tolist()) == res.resident
        info = gm.gnn_dyn_cache_query(fs)
        assert info["steps"] == ref.steps and info["refreshes"] == ref.refreshes
    assert ref.refreshes == 3      # after the calls that end at mini-batches 8, 16 and 24
    fs.close()


def test_three_streams_joined_around_the_refresh(tiny):
    """Super-batches on three streams (as the benchmark issues them), the streams joined before
    each refresh: rows stay exact and the policy matches the oracle's in host call order."""
    cfg, indptr, indices, x, order = tiny
    N, d, G, batch = cfg.num_nodes, cfg.d, 2, 512
    dg = device_graph(indptr, indices)
    fs = gm.gnn_feature_store_create(device_table(x, cfg.ld), d)
    K, T, gamma = 300, 6, 0.85
    gm.gnn_feature_store_enable_dynamic(fs, gamma, K, T)
    ref = oracle.DynCache(N, [], gamma, K, T)
    res = Residency()
    streams = [torch.cuda.Stream() for _ in range(3)]
    caps = gm.gnn_capacity(batch, cfg.fanouts, N)
    wss = [torch.empty(gm.gnn_workspace_size(caps, N, G), dtype=torch.uint8, device="cuda")
           for _ in streams]
    snap = None
    for window in range(3):
        issued = []
        for q, s in enumerate(streams):
            call = window * 3 + q
            lo = (call * G * batch) % (order.size - G * batch)
            seeds = order[lo:lo + G * batch]
            ptr = [0, batch, 2 * batch]
            outs = [gm.MinibatchOut(caps, d, cfg.ld, stream=s) for _ in range(G)]
            seed64 = gm.gnn_batch_seed(cfg.rng_seed, 100 + call)
            seeds_t = torch.from_numpy(seeds).cuda()    # kept alive until the join
            s.wait_stream(torch.cuda.current_stream())  # the seeds' copy, before the side stream reads them
            gm.gnn_minibatch(dg, fs, seeds_t, ptr, cfg.fanouts, seed64, outs, wss[q], None,
                             stream=s)
            issued.append((seeds, ptr, seed64, outs, seeds_t))
        torch.cuda.synchronize()    # the join
        for seeds, ptr, seed64, outs, _ in issued:
            refs = oracle.superbatch(indptr, indices, x, seeds, ptr, cfg.fanouts, seed64)
            for g in range(G):
                compare_with_oracle(outs[g], refs[g], d)
                ref.observe(refs[g].blocks[-1].nodes)
                res.gathered(refs[g].blocks[-1].nodes)
        for w in wss:
            assert gm.gnn_read_device_status(w) == gm.GNN_OK
        did = gm.gnn_dyn_cache_update(fs, stream=streams[0])
        assert did == ref.update()
        torch.cuda.synchronize()
        score, members, resident = device_state(fs, N)
        if did:
            snap = ref.score.copy()
            res.refreshed(members)
        np.testing.assert_allclose(score, ref.score, rtol=RTOL, atol=0)
        if snap is not None:
            check_members(members, snap, ref.is_static, K)
        assert set(resident.tolist()) == res.resident
    assert ref.refreshes == 3 and res.resident
    fs.close()


def test_enable_rejects_bad_parameters():
    x = torch.zeros(100, 4, device="cuda")
    hot = torch.arange(60, dtype=torch.int32, device="cuda")
    fs = gm.gnn_feature_store_create(x, 4, 60, hot)
    for kw in [dict(gamma=0.0, k_dyn=10, t_update=1), dict(gamma=1.0, k_dyn=10, t_update=1),
               dict(gamma=0.5, k_dyn=0, t_update=1), dict(gamma=0.5, k_dyn=41, t_update=1),
               dict(gamma=0.5, k_dyn=10, t_update=0), dict(gamma=0.5, k_dyn=10, t_update=1,
                                                           max_refreshes=-1)]:
        with pytest.raises(gm.GnnError):
            gm.gnn_feature_store_enable_dynamic(fs, **kw)
    with pytest.raises(gm.GnnError):
        gm.gnn_dyn_cache_update(fs)          # not enabled
    gm.gnn_feature_store_enable_dynamic(fs, 0.5, 40, 1)
    with pytest.raises(gm.GnnError):
        gm.gnn_feature_store_enable_dynamic(fs, 0.5, 10, 1)   # already enabled
    fs.close()
