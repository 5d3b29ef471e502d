"""graph_mini_pipeline_amd -- Python binding of libgnnmb.so, the MI355X (gfx950) GNN mini-batch path.

Argument marshalling only: torch tensors become device pointers and the current torch stream
becomes the hipStream_t.  Every step of the path (sampling, relabel, gather, aggregation) runs in
the library's HIP kernels; torch supplies device memory and streams.  The functions carry the C
names of include/gnnmb.h and raise GnnError on a negative status.
"""
from __future__ import annotations

import contextlib
import ctypes
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

from . import _abi
from ._abi import (GNN_ERR_CAPACITY, GNN_ERR_HIP, GNN_ERR_INTERNAL, GNN_ERR_INVALID_ARG,  # noqa
                   GNN_ERR_OUT_OF_RANGE, GNN_ERR_UNSUPPORTED, GNN_MAX_HOPS, GNN_OK, GNN_SYNC,
                   GNN_SUPERBATCH_COMPACT, GNN_SUPERBATCH_FULL, GNN_GATHER_BATCHED,
                   GNN_NOALLOC_MAX_IDS, GNN_NOALLOC_SCRATCH_BYTES, GNN_RELABEL_SORT, GNN_RELABEL_BITMAP, GNN_SAMPLE_EXACT_RANK,
                   GNN_GATHER_INTERLEAVED,
                   GNN_TIMER_STAGES)

__all__ = [
    "GnnError", "DeviceGraph", "Blocks", "MinibatchOut", "FeatureStore", "Timer", "Options",
    "gnn_status_string", "gnn_batch_seed", "gnn_capacity", "gnn_workspace_size", "gnn_sample_khop",
    "gnn_unique_relabel", "gnn_relabel_workspace_size", "gnn_feature_store_create",
    "gnn_feature_store_destroy", "gnn_gather_features", "gnn_mean_aggregate", "gnn_sage_layer",
    "gnn_sage_update", "gnn_minibatch", "gnn_unique_relabel_noalloc", "AdjacencyCache", "gnn_adjacency_cache_create",
    "gnn_host_mapped_pointer",
    "gnn_read_device_status", "gnn_timer_create", "gnn_timer_destroy", "gnn_timer_reset",
    "gnn_timer_elapsed", "gnn_copy_probe", "gnn_copy_probe_host", "gnn_hash_probe", "lib",
]

lib = _abi.lib


class GnnError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {gnn_status_string(status)} ({status})")


def _ok(status: int, what: str) -> None:
    if status != GNN_OK:
        raise GnnError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need(t: torch.Tensor, dtype, name: str, device=True) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")


def gnn_status_string(status: int) -> str:
    return lib().gnn_status_string(status).decode()


def gnn_batch_seed(rng_seed: int, b: int) -> int:
    return int(lib().gnn_batch_seed(rng_seed & 0xFFFFFFFFFFFFFFFF, b))


@dataclass
class Options:
    group_max_deg: int = 0
    wave_max_deg: int = 0
    sync: bool = False
    superbatch: str = "auto"    # super-batch relabel: "auto", "full" or "compact"
    gather: str = "auto"        # gather and outermost mean: "auto", "interleaved" or "batched"
    relabel: str = "auto"       # short id lists: "auto", "sort" (whenever eligible) or "bitmap"
    exact_rank: bool = False    # rank every node's candidates by the full (key, position) order
    d_hits: Optional[torch.Tensor] = None   # int64 [1] device: rows read from the HBM caches

    def c(self) -> _abi.gnn_options:
        o = _abi.gnn_options()
        if self.d_hits is not None:
            _need(self.d_hits, torch.int64, "d_hits")
            o.d_hits = self.d_hits.data_ptr()
        o.group_max_deg = self.group_max_deg
        o.wave_max_deg = self.wave_max_deg
        modes = {"auto": 0, "full": GNN_SUPERBATCH_FULL, "compact": GNN_SUPERBATCH_COMPACT}
        if self.superbatch not in modes:
            raise ValueError(f"superbatch must be one of {sorted(modes)}")
        gmodes = {"auto": 0, "interleaved": GNN_GATHER_INTERLEAVED, "batched": GNN_GATHER_BATCHED}
        if self.gather not in gmodes:
            raise ValueError(f"gather must be one of {sorted(gmodes)}")
        rmodes = {"auto": 0, "sort": GNN_RELABEL_SORT, "bitmap": GNN_RELABEL_BITMAP}
        if self.relabel not in rmodes:
            raise ValueError(f"relabel must be one of {sorted(rmodes)}")
        o.flags = (GNN_SYNC if self.sync else 0) | modes[self.superbatch] | gmodes[self.gather] | \
            rmodes[self.relabel] | (GNN_SAMPLE_EXACT_RANK if self.exact_rank else 0)
        return o


def gnn_host_mapped_pointer(t: torch.Tensor) -> int:
    """The device address of a pinned host tensor's memory."""
    if t.is_cuda or not t.is_pinned():
        raise ValueError("expected a pinned host tensor")
    out = ctypes.c_void_p()
    _ok(lib().gnn_host_mapped_pointer(_ptr(t), ctypes.byref(out)), "gnn_host_mapped_pointer")
    return int(out.value)


@dataclass
class DeviceGraph:
    """CSR by destination: indptr (int32 or int64) in device memory; indices (int32) in device
    memory or in pinned host memory (read in place); optionally an HBM adjacency cache."""
    num_nodes: int
    indptr: torch.Tensor
    indices: torch.Tensor
    adjacency: Optional["AdjacencyCache"] = None

    def c(self) -> _abi.gnn_graph:
        host = not self.indices.is_cuda
        _need(self.indices, torch.int32, "indices", device=not host)
        if host and self.indices.numel() and not self.indices.is_pinned():
            raise ValueError("host-resident indices must be pinned")
        if self.indptr.dtype not in (torch.int32, torch.int64) or not self.indptr.is_cuda:
            raise TypeError("indptr: int32 or int64 device tensor")
        g = _abi.gnn_graph()
        g.num_nodes = self.num_nodes
        g.num_edges = self.indices.numel()
        g.indptr = self.indptr.data_ptr()
        g.indptr_bytes = self.indptr.element_size()
        if not self.indices.numel():
            g.indices = None
        elif host:
            g.indices = gnn_host_mapped_pointer(self.indices)
        else:
            g.indices = self.indices.data_ptr()
        if self.adjacency is not None:
            _ok(lib().gnn_adjacency_cache_attach(self.adjacency.handle, ctypes.byref(g)),
                "gnn_adjacency_cache_attach")
        return g


class AdjacencyCache:
    """Owns a gnn_adjacency_cache handle (the HBM copies of hot adjacency rows)."""

    def __init__(self, handle: ctypes.c_void_p, rows: int, entries: int):
        self.handle = handle
        self.rows = rows
        self.entries = entries

    def close(self):
        if self.handle:
            lib().gnn_adjacency_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gnn_adjacency_cache_create(graph: DeviceGraph, hot_order: torch.Tensor,
                               max_entries: int) -> AdjacencyCache:
    """HBM copies of the rows of hot_order (device int32, hottest first) that fit max_entries
    neighbour ids; attach it with DeviceGraph(..., adjacency=cache)."""
    _need(hot_order, torch.int32, "hot_order")
    bare = DeviceGraph(graph.num_nodes, graph.indptr, graph.indices)
    g = bare.c()
    h = ctypes.c_void_p()
    rows, entries = ctypes.c_int64(), ctypes.c_int64()
    _ok(lib().gnn_adjacency_cache_create(ctypes.byref(g), _ptr(hot_order), hot_order.numel(),
                                         max_entries, ctypes.byref(h), ctypes.byref(rows),
                                         ctypes.byref(entries)),
        "gnn_adjacency_cache_create")
    return AdjacencyCache(h, rows.value, entries.value)


def gnn_capacity(n_seeds: int, fanouts: Sequence[int], num_nodes: int) -> _abi.gnn_caps:
    caps = _abi.gnn_caps()
    fo = (ctypes.c_int32 * len(fanouts))(*fanouts)
    _ok(lib().gnn_capacity(n_seeds, fo, len(fanouts), num_nodes, ctypes.byref(caps)), "gnn_capacity")
    return caps


def gnn_workspace_size(caps: _abi.gnn_caps, num_nodes: int, group: int = 1) -> int:
    n = ctypes.c_size_t(0)
    _ok(lib().gnn_workspace_size(ctypes.byref(caps), num_nodes, group, ctypes.byref(n)),
        "gnn_workspace_size")
    return int(n.value)


def gnn_relabel_workspace_size(id_bound: int) -> int:
    n = ctypes.c_size_t(0)
    _ok(lib().gnn_relabel_workspace_size(id_bound, ctypes.byref(n)), "gnn_relabel_workspace_size")
    return int(n.value)


class Blocks:
    """Device buffers of the K blocks of one batch, allocated at the given caps."""

    def __init__(self, caps: _abi.gnn_caps, device="cuda", stream=None):
        """`stream`: the stream the blocks are first written on.  The counts are zeroed by a kernel
        queued on it, so that the zeroing is ordered before that stream's calls (queued on the
        current stream instead, it could run after the counts of a call on a non-blocking side
        stream, and wipe them)."""
        self.caps = caps
        K = caps.num_hops
        i32 = torch.int32
        with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
            self.counts = torch.zeros(2 * K, dtype=torch.int64, device=device)
            self.indptr, self.gid, self.lid, self.dst_lid, self.nodes = [], [], [], [], []
            for l in range(K):
                self.indptr.append(torch.empty(caps.frontier[l] + 1, dtype=i32, device=device))
                self.gid.append(torch.empty(max(caps.edges[l], 1), dtype=i32, device=device))
                self.lid.append(torch.empty(max(caps.edges[l], 1), dtype=i32, device=device))
                self.dst_lid.append(torch.empty(max(caps.frontier[l], 1), dtype=i32, device=device))
                self.nodes.append(torch.empty(max(caps.nodes[l], 1), dtype=i32, device=device))

    def c(self) -> _abi.gnn_blocks:
        b = _abi.gnn_blocks()
        b.caps = self.caps
        for l in range(self.caps.num_hops):
            h = b.hop[l]
            h.indptr = self.indptr[l].data_ptr()
            h.gid = self.gid[l].data_ptr()
            h.lid = self.lid[l].data_ptr()
            h.dst_lid = self.dst_lid[l].data_ptr()
            h.nodes = self.nodes[l].data_ptr()
        b.counts = self.counts.data_ptr()
        return b

    def host(self):
        """Per-hop (indptr, gid, lid, dst_lid, nodes) trimmed to the device counts (syncs)."""
        cnt = self.counts.cpu().tolist()
        out = []
        F = self.caps.n_seeds
        for l in range(self.caps.num_hops):
            E, V = cnt[2 * l], cnt[2 * l + 1]
            out.append((self.indptr[l][:F + 1].cpu().numpy(), self.gid[l][:E].cpu().numpy(),
                        self.lid[l][:E].cpu().numpy(), self.dst_lid[l][:F].cpu().numpy(),
                        self.nodes[l][:V].cpu().numpy()))
            F = V
        return out


def gnn_sample_khop(graph: DeviceGraph, seeds: torch.Tensor, fanouts: Sequence[int], seed64: int,
                    blocks: Blocks, ws: torch.Tensor, opts: Optional[Options] = None,
                    stream=None) -> int:
    _need(seeds, torch.int32, "seeds")
    g = graph.c()
    b = blocks.c()
    fo = (ctypes.c_int32 * len(fanouts))(*fanouts)
    o = opts.c() if opts else None
    st = lib().gnn_sample_khop(ctypes.byref(g), _ptr(seeds) if seeds.numel() else None,
                               seeds.numel(), fo, len(fanouts), seed64 & 0xFFFFFFFFFFFFFFFF,
                               ctypes.byref(b), _ptr(ws), ws.numel() * ws.element_size(),
                               ctypes.byref(o) if o else None, _stream(stream))
    _ok(st, "gnn_sample_khop")
    return st


def gnn_unique_relabel(keep: torch.Tensor, add: torch.Tensor, id_bound: int, uniq: torch.Tensor,
                       d_n_uniq: torch.Tensor, add_lid: torch.Tensor, keep_lid: torch.Tensor,
                       ws: torch.Tensor, d_n_add: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    for t, n in ((keep, "keep"), (add, "add"), (uniq, "uniq"), (add_lid, "add_lid"),
                 (keep_lid, "keep_lid")):
        _need(t, torch.int32, n)
    _need(d_n_uniq, torch.int64, "d_n_uniq")
    if add_lid.numel() < add.numel() or keep_lid.numel() < keep.numel():
        raise ValueError("add_lid / keep_lid shorter than add / keep")
    st = lib().gnn_unique_relabel(_ptr(keep), keep.numel(), _ptr(add), _ptr(d_n_add), add.numel(),
                                  id_bound, _ptr(uniq), uniq.numel(), _ptr(d_n_uniq), _ptr(add_lid),
                                  _ptr(keep_lid), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream))
    _ok(st, "gnn_unique_relabel")


def gnn_unique_relabel_noalloc(keep: torch.Tensor, add: torch.Tensor, id_bound: int,
                               uniq: torch.Tensor, d_n_uniq: torch.Tensor, add_lid: torch.Tensor,
                               keep_lid: torch.Tensor, d_status: Optional[torch.Tensor] = None,
                               d_n_add: Optional[torch.Tensor] = None, stream=None) -> None:
    """gnn_unique_relabel on the library's fixed per-GPU scratch (no workspace, no allocation;
    id_bound <= GNN_NOALLOC_MAX_IDS; calls that overlap on one GPU race)."""
    for t, n in ((keep, "keep"), (add, "add"), (uniq, "uniq"), (add_lid, "add_lid"),
                 (keep_lid, "keep_lid")):
        _need(t, torch.int32, n)
    _need(d_n_uniq, torch.int64, "d_n_uniq")
    if d_status is not None:
        _need(d_status, torch.int32, "d_status")
    if add_lid.numel() < add.numel() or keep_lid.numel() < keep.numel():
        raise ValueError("add_lid / keep_lid shorter than add / keep")
    st = lib().gnn_unique_relabel_noalloc(_ptr(keep), keep.numel(), _ptr(add), _ptr(d_n_add),
                                          add.numel(), id_bound, _ptr(uniq), uniq.numel(),
                                          _ptr(d_n_uniq), _ptr(add_lid), _ptr(keep_lid),
                                          _ptr(d_status), _stream(stream))
    _ok(st, "gnn_unique_relabel_noalloc")


class FeatureStore:
    """Owns a gnn_feature_store handle; keeps the table (and hot order) tensors alive."""

    def __init__(self, handle: ctypes.c_void_p, table: torch.Tensor, d: int, ld: int):
        self.handle = handle
        self.table = table
        self.d = d
        self.ld = ld

    def close(self):
        if self.handle:
            lib().gnn_feature_store_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gnn_feature_store_create(table: torch.Tensor, d: int, cache_rows: int = 0,
                             hot_order: Optional[torch.Tensor] = None) -> FeatureStore:
    """table: float32 [N, ld] on the device, or pinned host memory (table.is_pinned())."""
    on_host = not table.is_cuda
    if on_host and not table.is_pinned():
        raise ValueError("a host feature table must be pinned")
    _need(table, torch.float32, "table", device=not on_host)
    if hot_order is not None:
        _need(hot_order, torch.int32, "hot_order")
    h = ctypes.c_void_p()
    st = lib().gnn_feature_store_create(_ptr(table), 1 if on_host else 0, table.shape[0], d,
                                        table.shape[1], cache_rows, _ptr(hot_order),
                                        ctypes.byref(h))
    _ok(st, "gnn_feature_store_create")
    return FeatureStore(h, table, d, table.shape[1])


def gnn_feature_store_destroy(fs: FeatureStore) -> None:
    fs.close()


def gnn_feature_store_enable_dynamic(fs: FeatureStore, gamma: float, k_dyn: int, t_update: int,
                                     max_refreshes: int = 0, auto: bool = False) -> None:
    """GARDEN's Dynamic-Cache on the store: k_dyn more HBM rows for residual hot rows, ranked by
    the EWMA of their accesses (decay gamma) and refreshed every t_update mini-batches; frozen
    after max_refreshes refreshes (0: never).  auto: gathers refresh when due, on their stream."""
    p = _abi.gnn_dyn_cache_params(float(gamma), int(k_dyn), int(t_update), int(max_refreshes),
                                  _abi.GNN_DYN_AUTO if auto else 0)
    _ok(lib().gnn_feature_store_enable_dynamic(fs.handle, ctypes.byref(p)),
        "gnn_feature_store_enable_dynamic")
    fs.dynamic = dict(gamma=float(gamma), k_dyn=int(k_dyn), t_update=int(t_update),
                      max_refreshes=int(max_refreshes), auto=bool(auto))


def gnn_dyn_cache_update(fs: FeatureStore, d_status: Optional[torch.Tensor] = None,
                         stream=None) -> bool:
    """Refresh the Dynamic-Cache on the stream if one is due; True if it ran."""
    r = ctypes.c_int32(0)
    _ok(lib().gnn_dyn_cache_update(fs.handle, ctypes.byref(r), _ptr(d_status), _stream(stream)),
        "gnn_dyn_cache_update")
    return bool(r.value)


def gnn_dyn_cache_query(fs: FeatureStore) -> dict:
    """Dynamic-Cache counters (synchronises the device)."""
    info = _abi.gnn_dyn_cache_info()
    _ok(lib().gnn_dyn_cache_query(fs.handle, ctypes.byref(info)), "gnn_dyn_cache_query")
    return {name: getattr(info, name) for name, _ in info._fields_ if name != "reserved"}


def gnn_dyn_cache_state(fs: FeatureStore, score: Optional[torch.Tensor] = None,
                        member: Optional[torch.Tensor] = None, stream=None) -> None:
    """score: float64 [N] device (Score(v, t) after the last observed mini-batch); member: uint8
    [N] device (1: holds a Dynamic-Cache row)."""
    n = fs.table.shape[0]
    if score is not None:
        _need(score, torch.float64, "score")
        if score.numel() < n:
            raise ValueError("score: [num_nodes]")
    if member is not None:
        _need(member, torch.uint8, "member")
        if member.numel() < n:
            raise ValueError("member: [num_nodes]")
    _ok(lib().gnn_dyn_cache_state(fs.handle, _ptr(score), _ptr(member), _stream(stream)),
        "gnn_dyn_cache_state")


def gnn_gather_features(fs: FeatureStore, ids: torch.Tensor, out: torch.Tensor,
                        d_n: Optional[torch.Tensor] = None, d_hits: Optional[torch.Tensor] = None,
                        d_status: Optional[torch.Tensor] = None, stream=None) -> None:
    _need(ids, torch.int32, "ids")
    _need(out, torch.float32, "out")
    if out.dim() != 2 or out.shape[0] < ids.numel():
        raise ValueError("out: [>= len(ids), ld_out]")
    st = lib().gnn_gather_features(fs.handle, _ptr(ids), _ptr(d_n), ids.numel(), _ptr(out),
                                   out.shape[1], _ptr(d_hits), _ptr(d_status), _stream(stream))
    _ok(st, "gnn_gather_features")


def gnn_gather_features_match(fs: FeatureStore, ids: torch.Tensor, out: torch.Tensor,
                              prev_ids: torch.Tensor, prev_x: torch.Tensor, match: torch.Tensor,
                              d_n: Optional[torch.Tensor] = None,
                              d_prev_n: Optional[torch.Tensor] = None,
                              d_matched: Optional[torch.Tensor] = None,
                              d_hits: Optional[torch.Tensor] = None,
                              d_status: Optional[torch.Tensor] = None, stream=None) -> None:
    """gnn_gather_features, with the rows whose ids are in prev_ids (strictly ascending) copied from
    prev_x (row p = features of prev_ids[p]); match[i] receives p or -1."""
    _need(ids, torch.int32, "ids")
    _need(out, torch.float32, "out")
    _need(prev_ids, torch.int32, "prev_ids")
    _need(prev_x, torch.float32, "prev_x")
    _need(match, torch.int32, "match")
    if out.dim() != 2 or out.shape[0] < ids.numel() or match.numel() < ids.numel():
        raise ValueError("out: [>= len(ids), ld_out]; match: [>= len(ids)]")
    if prev_x.dim() != 2 or prev_x.shape[0] < prev_ids.numel():
        raise ValueError("prev_x: [>= len(prev_ids), ld_prev]")
    st = lib().gnn_gather_features_match(fs.handle, _ptr(ids), _ptr(d_n), ids.numel(), _ptr(out),
                                         out.shape[1], _ptr(prev_ids), _ptr(d_prev_n),
                                         prev_ids.numel(), _ptr(prev_x), prev_x.shape[1],
                                         _ptr(match), _ptr(d_matched), _ptr(d_hits),
                                         _ptr(d_status), _stream(stream))
    _ok(st, "gnn_gather_features_match")


def gnn_batch_overlap(lists: Sequence[torch.Tensor], out: torch.Tensor,
                      counts: Optional[Sequence[Optional[torch.Tensor]]] = None,
                      stream=None) -> None:
    """out[a * B + b] = |lists[a] ∩ lists[b]| (device int64 [B * B]); each list strictly ascending,
    counts[a] (device int64 [1]) its actual length if given, else the whole tensor."""
    B = len(lists)
    _need(out, torch.int64, "out")
    if out.numel() < B * B:
        raise ValueError("out: [B * B]")
    for t in lists:
        _need(t, torch.int32, "lists")
    ids = (ctypes.c_void_p * B)(*[t.data_ptr() if t.numel() else None for t in lists])
    dn = None
    if counts is not None:
        dn = (ctypes.c_void_p * B)(*[c.data_ptr() if c is not None else None for c in counts])
    n = (ctypes.c_int64 * B)(*[t.numel() for t in lists])
    _ok(lib().gnn_batch_overlap(ids, dn, n, B, _ptr(out), _stream(stream)), "gnn_batch_overlap")


def gnn_greedy_order(overlap, first: int = 0) -> List[int]:
    """Nearest-overlap-first order of B batches from their overlap matrix (host array-like B x B)."""
    import numpy as np
    m = np.ascontiguousarray(np.asarray(overlap, dtype=np.int64))
    B = m.shape[0]
    if m.shape != (B, B):
        raise ValueError("overlap: B x B")
    order = (ctypes.c_int32 * B)()
    _ok(lib().gnn_greedy_order(m.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), B, first, order),
        "gnn_greedy_order")
    return list(order)


def gnn_mean_aggregate(indptr: torch.Tensor, lid: torch.Tensor, src: torch.Tensor, d: int,
                       out: torch.Tensor, d_n_dst: Optional[torch.Tensor] = None,
                       d_status: Optional[torch.Tensor] = None, stream=None) -> None:
    _need(indptr, torch.int32, "indptr")
    _need(lid, torch.int32, "lid")
    _need(src, torch.float32, "src")
    _need(out, torch.float32, "out")
    n_dst = indptr.numel() - 1
    if out.shape[0] < n_dst:
        raise ValueError("out has fewer rows than destinations")
    st = lib().gnn_mean_aggregate(_ptr(indptr), _ptr(lid), lid.numel(), _ptr(d_n_dst), n_dst,
                                  _ptr(src), src.shape[1], src.shape[0], d, _ptr(out),
                                  out.shape[1], _ptr(d_status), _stream(stream))
    _ok(st, "gnn_mean_aggregate")


def gnn_sage_layer(indptr: torch.Tensor, lid: torch.Tensor, dst_lid: torch.Tensor,
                   src: torch.Tensor, d: int, W: torch.Tensor, bias: Optional[torch.Tensor],
                   relu: bool, agg: torch.Tensor, out: torch.Tensor,
                   d_n_dst: Optional[torch.Tensor] = None, d_status: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """One GraphSAGE-mean layer: agg = block means, out = act([src[dst_lid] || agg] @ W + bias).
    W: float32 [2d, d_out] contiguous; agg: [n_dst, >= d]; out: [n_dst, >= d_out]."""
    for t, n in ((indptr, "indptr"), (lid, "lid"), (dst_lid, "dst_lid")):
        _need(t, torch.int32, n)
    for t, n in ((src, "src"), (W, "W"), (agg, "agg"), (out, "out")):
        _need(t, torch.float32, n)
    if bias is not None:
        _need(bias, torch.float32, "bias")
    n_dst = indptr.numel() - 1
    if W.dim() != 2 or W.shape[0] != 2 * d or not W.is_contiguous():
        raise ValueError("W must be a contiguous [2d, d_out] tensor")
    d_out = W.shape[1]
    if bias is not None and bias.numel() < d_out:
        raise ValueError("bias shorter than d_out")
    if dst_lid.numel() < n_dst or agg.shape[0] < n_dst or out.shape[0] < n_dst:
        raise ValueError("dst_lid / agg / out have fewer rows than destinations")
    st = lib().gnn_sage_layer(_ptr(indptr), _ptr(lid), lid.numel(), _ptr(dst_lid), _ptr(d_n_dst),
                              n_dst, _ptr(src), src.shape[1], src.shape[0], d, _ptr(W),
                              _ptr(bias), d_out, 1 if relu else 0, _ptr(agg), agg.shape[1],
                              _ptr(out), out.shape[1], _ptr(d_status), _stream(stream))
    _ok(st, "gnn_sage_layer")


def gnn_sage_update(dst_lid: torch.Tensor, src: torch.Tensor, d: int, agg: torch.Tensor,
                    W: torch.Tensor, bias: Optional[torch.Tensor], relu: bool, out: torch.Tensor,
                    n_dst: Optional[int] = None, d_n_dst: Optional[torch.Tensor] = None,
                    d_status: Optional[torch.Tensor] = None, stream=None) -> None:
    """The UPDATE alone: out = act([src[dst_lid] || agg] @ W + bias) for n_dst rows (default:
    dst_lid.numel()); agg holds the means."""
    _need(dst_lid, torch.int32, "dst_lid")
    for t, n in ((src, "src"), (W, "W"), (agg, "agg"), (out, "out")):
        _need(t, torch.float32, n)
    if bias is not None:
        _need(bias, torch.float32, "bias")
    n = dst_lid.numel() if n_dst is None else n_dst
    if W.dim() != 2 or W.shape[0] != 2 * d or not W.is_contiguous():
        raise ValueError("W must be a contiguous [2d, d_out] tensor")
    d_out = W.shape[1]
    if bias is not None and bias.numel() < d_out:
        raise ValueError("bias shorter than d_out")
    if dst_lid.numel() < n or agg.shape[0] < n or out.shape[0] < n:
        raise ValueError("dst_lid / agg / out have fewer rows than destinations")
    st = lib().gnn_sage_update(_ptr(dst_lid), _ptr(d_n_dst), n, _ptr(src), src.shape[1],
                               src.shape[0], d, _ptr(agg), agg.shape[1], _ptr(W), _ptr(bias), d_out,
                               1 if relu else 0, _ptr(out), out.shape[1], _ptr(d_status),
                               _stream(stream))
    _ok(st, "gnn_sage_update")


class MinibatchOut:
    """Blocks plus X and h_0..h_{K-1} of one (sub-)batch."""

    def __init__(self, caps: _abi.gnn_caps, d: int, ld_h: Optional[int] = None, device="cuda",
                 stream=None):
        """`stream`: the stream the outputs are first written on (as for Blocks)."""
        self.blocks = Blocks(caps, device, stream)
        self.d = d
        self.ld_h = ld_h if ld_h is not None else (d + 3) // 4 * 4
        K = caps.num_hops
        f32 = torch.float32
        with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
            self.x = torch.empty(max(caps.nodes[K - 1], 1), self.ld_h, dtype=f32, device=device)
            self.h = [torch.empty(max(caps.n_seeds if l == 0 else caps.nodes[l - 1], 1), self.ld_h,
                                  dtype=f32, device=device) for l in range(K)]

    def c(self) -> _abi.gnn_minibatch_out:
        m = _abi.gnn_minibatch_out()
        m.blocks = self.blocks.c()
        m.x = self.x.data_ptr()
        for l, t in enumerate(self.h):
            m.h[l] = t.data_ptr()
        m.ld_h = self.ld_h
        return m


class Timer:
    def __init__(self, n_records: int):
        h = ctypes.c_void_p()
        _ok(lib().gnn_timer_create(n_records, ctypes.byref(h)), "gnn_timer_create")
        self.handle = h
        self.n_records = n_records

    def reset(self):
        _ok(lib().gnn_timer_reset(self.handle), "gnn_timer_reset")

    def elapsed(self):
        """List of per-call stage times in ms: [sample+relabel, gather, outer mean, other means]."""
        n = ctypes.c_int32(0)
        buf = (ctypes.c_float * (self.n_records * GNN_TIMER_STAGES))()
        _ok(lib().gnn_timer_elapsed(self.handle, ctypes.byref(n), buf), "gnn_timer_elapsed")
        k = GNN_TIMER_STAGES
        return [list(buf[r * k:(r + 1) * k]) for r in range(n.value)]

    def close(self):
        if self.handle:
            lib().gnn_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gnn_timer_create(n_records: int) -> Timer:
    return Timer(n_records)


def gnn_timer_destroy(t: Timer) -> None:
    t.close()


def gnn_timer_reset(t: Timer) -> None:
    t.reset()


def gnn_timer_elapsed(t: Timer):
    return t.elapsed()


def gnn_minibatch(graph: DeviceGraph, fs: FeatureStore, seeds: torch.Tensor,
                  batch_ptr: Sequence[int], fanouts: Sequence[int], seed64: int,
                  outs: List[MinibatchOut], ws: torch.Tensor, opts: Optional[Options] = None,
                  stream=None, timer: Optional[Timer] = None) -> int:
    _need(seeds, torch.int32, "seeds")
    G = len(batch_ptr) - 1
    if len(outs) != G:
        raise ValueError("one MinibatchOut per sub-batch")
    g = graph.c()
    bp = (ctypes.c_int64 * (G + 1))(*batch_ptr)
    fo = (ctypes.c_int32 * len(fanouts))(*fanouts)
    mo = (_abi.gnn_minibatch_out * G)(*[o.c() for o in outs])
    o = opts.c() if opts else None
    st = lib().gnn_minibatch(ctypes.byref(g), fs.handle, _ptr(seeds) if seeds.numel() else None,
                             bp, G, fo, len(fanouts), seed64 & 0xFFFFFFFFFFFFFFFF, mo, _ptr(ws),
                             ws.numel() * ws.element_size(), ctypes.byref(o) if o else None,
                             _stream(stream), timer.handle if timer else None)
    _ok(st, "gnn_minibatch")
    return st


def gnn_copy_probe(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Plain device copy of src into dst (same byte size) by k_copy_probe; calibrates counters."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _ok(lib().gnn_copy_probe(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "gnn_copy_probe")


def gnn_copy_probe_host(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """The same copy with src in pinned host memory, read in place over the host link."""
    if src.is_cuda or not src.is_pinned():
        raise ValueError("src must be a pinned host tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _ok(lib().gnn_copy_probe_host(_ptr(src), _ptr(dst), nbytes, _stream(stream)),
        "gnn_copy_probe_host")


def gnn_hash_probe(seed: int, tau: int, lanes: int, per_lane: int, d_count: torch.Tensor,
                   stream=None) -> None:
    """lanes * per_lane sampling keys (mix64 of a stepped counter); adds the keys <= tau to d_count."""
    _need(d_count, torch.int64, "d_count")
    _ok(lib().gnn_hash_probe(seed, tau, lanes, per_lane, _ptr(d_count), _stream(stream)),
        "gnn_hash_probe")


def gnn_read_device_status(ws: torch.Tensor, stream=None) -> int:
    out = ctypes.c_int32(0)
    _ok(lib().gnn_read_device_status(_ptr(ws), _stream(stream), ctypes.byref(out)),
        "gnn_read_device_status")
    return int(out.value)
