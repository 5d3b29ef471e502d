"""Hot-row ranking for the HBM feature cache, by pre-sampling (set-up, not on the mini-batch path).

The caches of the pages are filled offline from access statistics: GARDEN (Sec. II.B, the
Nfeat-cache of the Dual-Cache System; Sec. IV.B, Table III, a few pre-sampling epochs) profiles
which feature rows sampling touches; LEO (Sec. 2.3 and its related work) names degree-ranked and
pre-sampling-ranked hot caches.  Here P batches are sampled with the library's own sampler, each
node counts the batches whose gathered set V_K holds it, and rows are ranked by (count descending,
in-degree descending, id ascending).  The ranking only decides which rows sit in HBM: outputs are
the same for any ranking.  The batches should not be the measured ones (a disjoint seed stream).
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (Blocks, DeviceGraph, gnn_batch_seed, gnn_capacity, gnn_read_device_status,
               gnn_sample_khop, gnn_workspace_size, GNN_OK, GnnError)


def presample_counts(graph: DeviceGraph, seeds: torch.Tensor, batch: int, fanouts: Sequence[int],
                     rng_seed: int, levels: Optional[Sequence[int]] = None) -> torch.Tensor:
    """int32 [len(levels), N]: for each level l in `levels` and node v, the number of pre-sampled
    batches with v in V_l (V_0: the seeds); by default levels = [K] (the gathered set V_K) and the
    result is [N].  Batch p takes seeds[p*batch:(p+1)*batch] and the batch seed
    gnn_batch_seed(rng_seed, p)."""
    N = graph.num_nodes
    K = len(fanouts)
    dev = seeds.device
    lv_list = list(levels) if levels is not None else [K]
    counts = torch.zeros(len(lv_list), N, dtype=torch.int32, device=dev)
    caps = gnn_capacity(batch, fanouts, N)
    blocks = Blocks(caps)
    ws = torch.empty(gnn_workspace_size(caps, N), dtype=torch.uint8, device=dev)
    P = seeds.numel() // batch
    for p in range(P):
        s = seeds[p * batch:(p + 1) * batch].contiguous()
        gnn_sample_khop(graph, s, fanouts, gnn_batch_seed(rng_seed, p), blocks, ws)
        st = gnn_read_device_status(ws)
        if st != GNN_OK:
            raise GnnError(st, "pre-sampling")
        for j, lv in enumerate(lv_list):
            if lv == 0:
                ids = s
            else:
                ids = blocks.nodes[lv - 1][:int(blocks.counts[2 * lv - 1].item())]
            counts[j].index_add_(0, ids.long(),
                                 torch.ones(ids.numel(), dtype=torch.int32, device=dev))
    return counts if levels is not None else counts[0]


def rank_rows(counts: torch.Tensor, degree: torch.Tensor, rows: int,
              degree_desc: bool = True) -> torch.Tensor:
    """int32 [rows]: the ids of the `rows` hottest rows by (count desc, degree desc, id asc), or
    with degree_desc=False by (count desc, degree asc, id asc)."""
    N = counts.numel()
    id_bits = max(1, (N - 1).bit_length())
    cmax = int(counts.max().item()) if N else 0
    c_bits = max(1, cmax.bit_length())
    d_bits = 63 - id_bits - c_bits
    if d_bits < 1:
        raise ValueError("too many nodes or counts for the ranking key")
    dcap = (1 << d_bits) - 1
    ids = torch.arange(N, dtype=torch.int64, device=counts.device)
    dkey = degree.to(torch.int64).clamp(0, dcap)
    key = ((cmax - counts.to(torch.int64)) << (d_bits + id_bits)) \
        | ((dcap - dkey if degree_desc else dkey) << id_bits) | ids
    order = torch.sort(key).values & ((1 << id_bits) - 1)
    return order[:rows].to(torch.int32).contiguous()


def presample_hot_order(graph: DeviceGraph, indptr: torch.Tensor, seeds: torch.Tensor, batch: int,
                        fanouts: Sequence[int], rng_seed: int, rows: int) -> torch.Tensor:
    """Hot-row order for gnn_feature_store_create: pre-sample, count, rank (see module doc)."""
    counts = presample_counts(graph, seeds, batch, fanouts, rng_seed)
    degree = indptr[1:] - indptr[:-1]
    return rank_rows(counts, degree, rows)


def presample_adjacency_order(graph: DeviceGraph, indptr: torch.Tensor, seeds: torch.Tensor,
                              batch: int, fanouts: Sequence[int], rng_seed: int) -> torch.Tensor:
    """Hot order for gnn_adjacency_cache_create.  At hop l the sampler reads min(deg v, k_l) ids of
    node v's row when v is in the frontier V_{l-1} (GARDEN Sec. IV.B counts the accesses of the
    whole sampling path, eq. (4)).  A cached row costs deg v ids of HBM and saves, per pre-sampled
    batch, sum_l [v in V_{l-1}] * min(deg v, k_l) host reads; rows that save anything are ranked
    by saved reads per cached id (descending, then id ascending): a hub read k times out of
    thousands of ids ranks below a short row read whole."""
    K = len(fanouts)
    counts = presample_counts(graph, seeds, batch, fanouts, rng_seed, levels=list(range(K)))
    # rows the pre-sampling never reached follow, by how many rows list the node (the ways it can
    # be sampled into a frontier)
    outdeg = torch.bincount(graph.indices, minlength=graph.num_nodes).to(indptr.device)
    return rank_adjacency(counts, indptr[1:] - indptr[:-1], fanouts, outdeg)


def rank_adjacency(counts: torch.Tensor, degree: torch.Tensor, fanouts: Sequence[int],
                   outdeg: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32: the nodes whose cached rows save host reads, by saved reads per cached id
    sum_l counts[l, v] * min(deg v, k_{l+1}) / deg v, descending (ties: id ascending).
    counts: [K, N], counts[l, v] = batches whose frontier V_l holds v; degree: [N].  With outdeg
    ([N], the number of rows listing each node) the other non-empty rows follow by the estimate
    outdeg v * min(deg v, max k) / deg v, descending (ties: id ascending)."""
    degree = degree.to(torch.float64)
    saved = torch.zeros_like(degree)
    for l, k in enumerate(fanouts):
        saved += counts[l].to(torch.float64) * degree.clamp(max=k)
    density = saved / degree.clamp(min=1)
    live = torch.nonzero(saved > 0).flatten()
    # stable sort of the live ids (ascending) by density, descending: ties keep id order
    order = live[torch.sort(density[live], descending=True, stable=True).indices]
    if outdeg is not None:
        est = outdeg.to(torch.float64) * degree.clamp(max=max(fanouts)) / degree.clamp(min=1)
        rest = torch.nonzero((saved == 0) & (est > 0)).flatten()
        order = torch.cat([order, rest[torch.sort(est[rest], descending=True, stable=True).indices]])
    return order.to(torch.int32).contiguous()
