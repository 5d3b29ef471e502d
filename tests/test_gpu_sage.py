"""Parity of the GraphSAGE-mean layer (gnn_sage_layer) with the oracle.

The means must equal gnn_mean_aggregate's bit for bit (the same kernel) and the oracle's within
1e-5 * max|src|.  The layer output is an fp32 matrix-core product of 2d terms plus a bias; its
error against the oracle's double result is bounded per element by
    (2d + c_max + 8) * 2^-24 * (sum_k |a_k| |W_kn| + |b_n|),
the classical bound for a float dot product of 2d terms in any order (the mean's own rounding
error, at most (c + 1) ulps of the row scale, is covered by the c_max term).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

gm = pytest.importorskip("graph_mini_pipeline_amd")


def _tol(scale, d, c_max):
    return (2 * d + c_max + 8) * 2.0 ** -24 * scale


def _block(rng, n_dst, n_src, max_c):
    counts = rng.integers(0, max_c + 1, size=n_dst)
    if n_dst > 3:
        counts[[1, n_dst - 2]] = 0   # destinations without sampled neighbours
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    lid = rng.integers(0, n_src, size=int(counts.sum())).astype(np.int32)
    dst_lid = rng.integers(0, n_src, size=n_dst).astype(np.int32)
    return indptr, lid, dst_lid


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def _run(indptr, lid, dst_lid, src, ld_src, d, W, b, relu, ld_agg, ld_out, d_n_dst=None):
    n_dst = len(indptr) - 1
    src_t = torch.zeros(src.shape[0], ld_src, dtype=torch.float32, device="cuda")
    src_t[:, :d] = _dev(src)
    agg = torch.full((max(n_dst, 1), ld_agg), -7.0, dtype=torch.float32, device="cuda")
    out = torch.full((max(n_dst, 1), ld_out), -7.0, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    lid_t = _dev(lid) if lid.size else torch.zeros(1, dtype=torch.int32, device="cuda")[:0]
    gm.gnn_sage_layer(_dev(indptr), lid_t, _dev(dst_lid), src_t, d, _dev(W),
                      None if b is None else _dev(b), relu, agg, out, d_n_dst=d_n_dst,
                      d_status=status)
    torch.cuda.synchronize()
    return src_t, lid_t, agg, out, int(status.item())


CASES = [
    # n_dst, n_src, d, d_out, c_max, relu, bias, ld_src, ld_agg, ld_out
    (1, 3, 4, 16, 3, True, True, 4, 4, 16),
    (63, 100, 64, 64, 10, False, True, 64, 64, 64),
    (65, 90, 33, 17, 5, True, False, 36, 40, 20),       # unaligned rows, K not a chunk multiple
    (130, 400, 100, 100, 15, True, True, 100, 104, 100),
    (257, 600, 602, 128, 25, True, True, 604, 604, 128),  # the dense workload's row width
    (500, 900, 5, 200, 7, False, True, 8, 5, 203),      # K = 10 < one chunk, 4 N tiles
    (8300, 9000, 24, 256, 6, True, True, 24, 28, 256),  # enough tiles for 64-row tiles
]


@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}-d{c[2]}-o{c[3]}" for c in CASES])
def test_sage_layer_parity(case):
    n_dst, n_src, d, d_out, c_max, relu, has_b, ld_src, ld_agg, ld_out = case
    rng = np.random.default_rng(n_dst * 131 + d)
    indptr, lid, dst_lid = _block(rng, n_dst, n_src, c_max)
    src = rng.standard_normal((n_src, d)).astype(np.float32)
    W = (rng.standard_normal((2 * d, d_out)) / np.sqrt(2 * d)).astype(np.float32)
    b = rng.standard_normal(d_out).astype(np.float32) if has_b else None
    src_t, lid_t, agg, out, st = _run(indptr, lid, dst_lid, src, ld_src, d, W, b, relu, ld_agg,
                                      ld_out)
    assert st == gm.GNN_OK
    # the means: bit for bit those of gnn_mean_aggregate, within the aggregation bound of the oracle
    ref_mean = torch.full_like(agg, -7.0)
    gm.gnn_mean_aggregate(_dev(indptr), lid_t, src_t, d, ref_mean)
    torch.cuda.synchronize()
    assert torch.equal(agg[:n_dst, :d], ref_mean[:n_dst, :d])
    om = oracle.mean_aggregate(indptr, lid, src)
    scale = float(np.abs(src).max())
    assert float(np.abs(agg[:n_dst, :d].cpu().numpy() - om).max()) <= 1e-5 * scale
    # the layer
    ref, mag = oracle.sage_layer(indptr, lid, dst_lid, src, W, b, relu, with_scale=True)
    got = out[:n_dst, :d_out].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    tol = _tol(mag, d, c_max)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{len(bad)} outputs off, first {bad[:3].tolist()}, err {err.max()}"
    if relu:
        assert (got >= 0).all()
    # padding columns untouched
    if ld_out > d_out:
        assert (out[:n_dst, d_out:] == -7.0).all()


def test_sage_layer_device_count_and_empty():
    """Rows at or beyond *d_n_dst are left alone; an empty block enqueues nothing harmful."""
    rng = np.random.default_rng(5)
    indptr, lid, dst_lid = _block(rng, 150, 200, 6)
    src = rng.standard_normal((200, 16)).astype(np.float32)
    W = rng.standard_normal((32, 70)).astype(np.float32)
    d_n = torch.tensor([97], dtype=torch.int64, device="cuda")
    _, _, agg, out, st = _run(indptr, lid, dst_lid, src, 16, 16, W, None, False, 16, 70, d_n)
    assert st == gm.GNN_OK
    ref = oracle.sage_layer(indptr[:98], lid[:indptr[97]], dst_lid[:97], src, W, None, False)
    got = out[:97].cpu().numpy().astype(np.float64)
    mag = oracle.sage_layer(indptr[:98], lid[:indptr[97]], dst_lid[:97], np.abs(src),
                            np.abs(W), None, False)
    assert (np.abs(got - ref) <= _tol(mag, 16, 6)).all()
    assert (out[97:] == -7.0).all()
    e = np.zeros(1, np.int32)
    _, _, _, out0, st = _run(e, np.zeros(0, np.int32), np.zeros(0, np.int32), src, 16, 16, W,
                             None, True, 16, 70)
    assert st == gm.GNN_OK and (out0 == -7.0).all()


def test_sage_layer_rejects_bad_dst_lid():
    """A destination row outside src is reported on the status word (that row reads row 0)."""
    rng = np.random.default_rng(6)
    indptr, lid, dst_lid = _block(rng, 40, 50, 4)
    dst_lid[7] = 50
    src = rng.standard_normal((50, 8)).astype(np.float32)
    W = rng.standard_normal((16, 8)).astype(np.float32)
    _, _, _, _, st = _run(indptr, lid, dst_lid, src, 8, 8, W, None, False, 8, 8)
    assert st == gm.GNN_ERR_INTERNAL


def test_sage_layer_on_dense_outermost_block():
    """The dense workload (602-d rows, fanouts [25, 10]): one batch's outermost block through a
    128-wide layer, checked on sampled destinations against the oracle."""
    cfg = synth.CONFIGS["dense"]
    dev = torch.device("cuda")
    g = synth.build_graph(cfg, device=dev)
    table = torch.empty(cfg.num_nodes, cfg.ld, dtype=torch.float32, device=dev)
    synth.make_features(cfg, table)
    order = synth.epoch_seed_order(cfg, 0, device=dev).contiguous()
    dg = gm.DeviceGraph(cfg.num_nodes, g.indptr, g.indices)
    fs = gm.gnn_feature_store_create(table, cfg.d)
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, cfg.num_nodes)
    mo = gm.MinibatchOut(caps, cfg.d, cfg.ld)
    ws = torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes, 1), dtype=torch.uint8, device=dev)
    gm.gnn_minibatch(dg, fs, order[:cfg.batch].contiguous(), [0, cfg.batch], cfg.fanouts,
                     gm.gnn_batch_seed(cfg.rng_seed, 0), [mo], ws)
    torch.cuda.synchronize()
    K = len(cfg.fanouts)
    blk = mo.blocks.host()[K - 1]
    ind, gid, lid, dst_lid, nodes = blk
    n_dst = len(ind) - 1
    nv = len(nodes)
    d_out = 128
    gen = torch.Generator().manual_seed(11)
    W = (torch.randn(2 * cfg.d, d_out, generator=gen) / np.sqrt(2 * cfg.d)).to(torch.float32)
    b = torch.randn(d_out, generator=gen).to(torch.float32)
    agg = torch.empty(n_dst, cfg.ld, dtype=torch.float32, device=dev)
    out = torch.empty(n_dst, d_out, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    gm.gnn_sage_layer(_dev(ind), _dev(lid), _dev(dst_lid), mo.x, cfg.d, W.cuda(), b.cuda(), True,
                      agg, out, d_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == gm.GNN_OK
    x = mo.x[:nv, :cfg.d].cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, n_dst, max(1, n_dst // 300)), [n_dst - 1]]))
    counts = ind[rows + 1] - ind[rows]
    sub_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sub_lid = np.concatenate([lid[ind[r]:ind[r + 1]] for r in rows]).astype(np.int32)
    ref, mag = oracle.sage_layer(sub_ptr, sub_lid, dst_lid[rows], x, W.numpy(), b.numpy(), True,
                                 with_scale=True)
    got = out[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) <= _tol(mag, cfg.d, max(cfg.fanouts))).all()
    # the UPDATE alone on the means gnn_minibatch computed (h_{K-1}) gives the same bits
    h = mo.h[K - 1]
    assert torch.equal(h[:n_dst, :cfg.d], agg[:n_dst, :cfg.d])
    out2 = torch.empty_like(out)
    gm.gnn_sage_update(_dev(dst_lid), mo.x, cfg.d, h, W.cuda(), b.cuda(), True, out2,
                       d_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == gm.GNN_OK
    assert torch.equal(out2, out)
