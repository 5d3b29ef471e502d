"""GPU-test helpers: run the HIP path through the binding and compare it with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import graph_mini_pipeline_amd as gm
import oracle


def device_graph(indptr: np.ndarray, indices: np.ndarray) -> gm.DeviceGraph:
    n = indptr.shape[0] - 1
    ind = torch.from_numpy(np.ascontiguousarray(indices, dtype=np.int32)).cuda()
    if ind.numel() == 0:
        ind = torch.zeros(1, dtype=torch.int32, device="cuda")[:0]
    return gm.DeviceGraph(n, torch.from_numpy(np.ascontiguousarray(indptr)).cuda(), ind)


def device_table(x: np.ndarray, ld: int) -> torch.Tensor:
    n, d = x.shape
    t = torch.zeros(n, ld, dtype=torch.float32, device="cuda")
    t[:, :d] = torch.from_numpy(x).cuda()
    return t


def run_minibatch(dg: gm.DeviceGraph, fs: gm.FeatureStore, seeds: np.ndarray, fanouts, seed64,
                  opts=None, ws=None, group_ptr=None):
    """Run gnn_minibatch; returns (outs, status).  group_ptr splits seeds into sub-batches."""
    seeds_t = torch.from_numpy(np.ascontiguousarray(seeds, dtype=np.int32)).cuda()
    ptr = group_ptr if group_ptr is not None else [0, len(seeds)]
    outs = []
    caps_max = None
    for g in range(len(ptr) - 1):
        caps = gm.gnn_capacity(ptr[g + 1] - ptr[g], fanouts, dg.num_nodes)
        outs.append(gm.MinibatchOut(caps, fs.d, fs.ld))
        if caps_max is None or caps.frontier[len(fanouts) - 1] > caps_max.frontier[len(fanouts) - 1]:
            caps_max = caps
    if ws is None:
        need = max(gm.gnn_workspace_size(o.blocks.caps, dg.num_nodes, len(ptr) - 1) for o in outs)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    gm.gnn_minibatch(dg, fs, seeds_t, ptr, fanouts, seed64, outs, ws, opts)
    st = gm.gnn_read_device_status(ws)
    return outs, st


def compare_with_oracle(out: gm.MinibatchOut, ref: oracle.MiniBatch, d: int, tol_scale=1e-5):
    """Bit-exact blocks and X; h within tol_scale * max|X| per layer."""
    got = out.blocks.host()
    K = len(ref.blocks)
    for l in range(K):
        ind, gid, lid, dst, nodes = got[l]
        rb = ref.blocks[l]
        assert np.array_equal(ind, rb.indptr), f"hop {l + 1}: block indptr"
        assert np.array_equal(gid, rb.gid), f"hop {l + 1}: sampled ids"
        assert np.array_equal(nodes, rb.nodes), f"hop {l + 1}: V_l"
        assert np.array_equal(lid, rb.lid), f"hop {l + 1}: lid"
        assert np.array_equal(dst, rb.dst_lid), f"hop {l + 1}: dst_lid"
    nv = len(ref.blocks[-1].nodes)
    x = out.x[:nv, :d].cpu().numpy()
    assert np.array_equal(x.view(np.uint32), ref.x.view(np.uint32)), "gathered rows"
    scale = float(np.abs(ref.x).max()) if ref.x.size else 1.0
    tol = tol_scale * max(scale, 1e-30)
    for l in range(K):
        rows = ref.h[l].shape[0]
        h = out.h[l][:rows, :d].cpu().numpy()
        err = float(np.abs(h.astype(np.float64) - ref.h[l]).max()) if rows else 0.0
        assert err <= tol, f"h_{l}: max err {err} > {tol}"
