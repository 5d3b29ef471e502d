"""The allocation-free relabel (gnn_unique_relabel_noalloc, scratch in a fixed per-GPU array)
against the workspace entry point gnn_unique_relabel, through the C ABI: two calls in a row, the
second smaller (the scratch keeps the first call's contents), bit for bit."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

gm = pytest.importorskip("graph_mini_pipeline_amd")


def _lists(rng, id_bound, n_keep, n_add):
    keep = rng.choice(id_bound, size=n_keep, replace=False).astype(np.int32)
    add = rng.integers(0, id_bound, size=n_add, dtype=np.int64).astype(np.int32)
    add[: n_add // 4] = rng.choice(keep, size=n_add // 4)      # ids shared with keep
    return keep, add


def _run(fn, keep, add, id_bound, **kw):
    dev = lambda a: torch.from_numpy(a).cuda()
    n = len(keep) + len(add)
    uniq = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int64, device="cuda")
    add_lid = torch.full((len(add),), -7, dtype=torch.int32, device="cuda")
    keep_lid = torch.full((len(keep),), -7, dtype=torch.int32, device="cuda")
    fn(dev(keep), dev(add), id_bound, uniq, nu, add_lid, keep_lid, **kw)
    torch.cuda.synchronize()
    m = int(nu.item())
    return uniq[:m].cpu().numpy(), add_lid.cpu().numpy(), keep_lid.cpu().numpy()


def _with_ws(keep, add, id_bound):
    ws = torch.empty(gm.gnn_relabel_workspace_size(id_bound), dtype=torch.uint8, device="cuda")

    def fn(*a):
        gm.gnn_unique_relabel(*a, ws)
    got = _run(fn, keep, add, id_bound)
    assert gm.gnn_read_device_status(ws) == gm.GNN_OK
    return got


def test_noalloc_equals_workspace_entry_point_twice():
    rng = np.random.default_rng(20261202)
    # first call at the largest id range the scratch holds, the second much smaller
    for id_bound, n_keep, n_add in ((gm.GNN_NOALLOC_MAX_IDS, 20_000, 400_000), (50_000, 1000, 8000)):
        keep, add = _lists(rng, id_bound, n_keep, n_add)
        status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
        got = _run(gm.gnn_unique_relabel_noalloc, keep, add, id_bound, d_status=status)
        assert int(status.item()) == gm.GNN_OK
        ref = _with_ws(keep, add, id_bound)
        for g, r, name in zip(got, ref, ("uniq", "add_lid", "keep_lid")):
            assert np.array_equal(g, r), name
        assert np.array_equal(got[0], np.unique(np.concatenate([keep, add])))


def test_noalloc_device_count_and_status():
    rng = np.random.default_rng(7)
    keep, add = _lists(rng, 10_000, 300, 2000)
    n_add = torch.tensor([1500], dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = _run(gm.gnn_unique_relabel_noalloc, keep, add, 10_000, d_status=status, d_n_add=n_add)
    assert int(status.item()) == gm.GNN_OK
    assert np.array_equal(got[0], np.unique(np.concatenate([keep, add[:1500]])))
    assert np.array_equal(got[0][got[1][:1500]], add[:1500])
    # an id at the bound is reported on the status word (the kernels skip it)
    bad = add.copy()
    bad[5] = 10_000
    _run(gm.gnn_unique_relabel_noalloc, keep, bad, 10_000, d_status=status)
    assert int(status.item()) == gm.GNN_ERR_OUT_OF_RANGE
