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


def oracle_pool(indptr, indices, x, d, jobs, threads=None):
    """Oracle results of many batches, computed concurrently on host threads (the oracle's C
    calls release the interpreter lock; no process is forked from this GPU process).
    jobs: iterable of (key, seeds, fanouts, seed64).  Returns (executor, {key: future})."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    oracle.lib()      # load once, before the threads start
    n = threads or max(1, min(16, os.cpu_count() or 1))
    ex = ThreadPoolExecutor(max_workers=n)
    futs = {key: ex.submit(oracle.minibatch, indptr, indices, x, np.ascontiguousarray(seeds),
                           list(fanouts), seed64, d=d)
            for key, seeds, fanouts, seed64 in jobs}
    return ex, futs


def headline_layout(cfg, dg, fs, order, steps, G, P=3, rounds=1, opts=None):
    """Super-batches issued the way the benchmark's headline issues them: step st (super-batch st
    of the seed order `order`, batch seed gnn_batch_seed(rng_seed, st)) goes to stream i % P of a
    window of P * rounds steps, each stream with a workspace of its own, and each (stream, round)
    with output sets of its own, so `rounds` steps run back to back on every stream while the
    other streams run theirs; the host synchronises once per window.  Output sets are reused by
    the next window.  Yields (st, b, seed64, out) for every sub-batch b of every step."""
    import math
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, cfg.num_nodes)
    streams = [torch.cuda.Stream() for _ in range(P)]
    wss = [torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes, G), dtype=torch.uint8,
                       device="cuda") for _ in range(P)]
    n_batches = math.ceil(order.numel() / cfg.batch)
    sets = {}
    steps = list(steps)
    window = P * rounds
    for w0 in range(0, len(steps), window):
        issued = []
        for i, st in enumerate(steps[w0:w0 + window]):
            q, r = i % P, i // P
            bs = list(range(st * G, min(st * G + G, n_batches)))
            lo = bs[0] * cfg.batch
            hi = min(order.numel(), (bs[-1] + 1) * cfg.batch)
            ptr = [b * cfg.batch - lo for b in bs] + [hi - lo]
            outs = []
            for j in range(len(bs)):
                n = ptr[j + 1] - ptr[j]
                key = (q, r, j, n)
                if key not in sets:
                    sets[key] = gm.MinibatchOut(gm.gnn_capacity(n, cfg.fanouts, cfg.num_nodes),
                                                cfg.d, cfg.ld, stream=streams[q])
                outs.append(sets[key])
            seed64 = gm.gnn_batch_seed(cfg.rng_seed, st)
            gm.gnn_minibatch(dg, fs, order[lo:hi], ptr, cfg.fanouts, seed64, outs, wss[q], opts,
                             stream=streams[q])
            issued.append((st, bs, seed64, outs))
        torch.cuda.synchronize()
        for w in wss:
            assert gm.gnn_read_device_status(w) == gm.GNN_OK
        for st, bs, seed64, outs in issued:
            for b, out in zip(bs, outs):
                yield st, b, seed64, out
