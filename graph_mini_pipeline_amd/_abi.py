"""ctypes mirror of include/gnnmb.h and the loader of libgnnmb.so.

Loading fails loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgnnmb.so")

GNN_MAX_HOPS = 8
GNN_MAX_GROUP = 16
GNN_TIMER_STAGES = 5
GNN_SYNC = 1
GNN_SUPERBATCH_FULL = 2
GNN_SUPERBATCH_COMPACT = 4
GNN_GATHER_INTERLEAVED = 8
GNN_GATHER_BATCHED = 16
GNN_RELABEL_SORT = 32
GNN_RELABEL_BITMAP = 64
GNN_SAMPLE_EXACT_RANK = 128
GNN_NOALLOC_MAX_IDS = 1 << 26
GNN_NOALLOC_SCRATCH_BYTES = (24 << 20) + (64 << 10)
GNN_DYN_AUTO = 1

GNN_OK = 0
GNN_ERR_INVALID_ARG = -1
GNN_ERR_CAPACITY = -2
GNN_ERR_OUT_OF_RANGE = -3
GNN_ERR_HIP = -4
GNN_ERR_UNSUPPORTED = -5
GNN_ERR_INTERNAL = -6

i32, i64, u32, u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p
size_t = ctypes.c_size_t


class gnn_graph(ctypes.Structure):
    _fields_ = [("num_nodes", i64), ("num_edges", i64), ("indptr", vp), ("indptr_bytes", i32),
                ("indices", vp), ("adj_off", vp), ("adj_rows", vp)]


class gnn_caps(ctypes.Structure):
    _fields_ = [("num_hops", i32), ("fanouts", i32 * GNN_MAX_HOPS), ("n_seeds", i64),
                ("frontier", i64 * GNN_MAX_HOPS),
                ("edges", i64 * GNN_MAX_HOPS), ("nodes", i64 * GNN_MAX_HOPS)]


class gnn_block(ctypes.Structure):
    _fields_ = [("indptr", vp), ("gid", vp), ("lid", vp), ("dst_lid", vp), ("nodes", vp)]


class gnn_blocks(ctypes.Structure):
    _fields_ = [("caps", gnn_caps), ("hop", gnn_block * GNN_MAX_HOPS), ("counts", vp)]


class gnn_options(ctypes.Structure):
    _fields_ = [("group_max_deg", i32), ("wave_max_deg", i32), ("flags", u32),
                ("reserved0", i32), ("d_hits", vp), ("reserved", i32 * 2)]


class gnn_dyn_cache_params(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_double), ("k_dyn", i64), ("t_update", i32),
                ("max_refreshes", i32), ("flags", u32)]


class gnn_dyn_cache_info(ctypes.Structure):
    _fields_ = [("steps", i64), ("since_refresh", i64), ("refreshes", i32), ("due", i32),
                ("frozen", i32), ("reserved", i32), ("members", i64), ("last_candidates", i64),
                ("last_admitted", i64), ("last_evicted", i64), ("resident", i64),
                ("last_published", i64)]


class gnn_minibatch_out(ctypes.Structure):
    _fields_ = [("blocks", gnn_blocks), ("x", vp), ("h", vp * GNN_MAX_HOPS), ("ld_h", i64)]


P = ctypes.POINTER

# name -> (restype, argtypes); every entry point the header declares
SIGNATURES = {
    "gnn_status_string": (ctypes.c_char_p, [i32]),
    "gnn_batch_seed": (u64, [u64, u64]),
    "gnn_capacity": (i32, [i64, P(i32), i32, i64, P(gnn_caps)]),
    "gnn_workspace_size": (i32, [P(gnn_caps), i64, i32, P(size_t)]),
    "gnn_sample_khop": (i32, [P(gnn_graph), vp, i64, P(i32), i32, u64, P(gnn_blocks), vp, size_t,
                              P(gnn_options), vp]),
    "gnn_unique_relabel": (i32, [vp, i64, vp, vp, i64, i64, vp, i64, vp, vp, vp, vp, size_t, vp]),
    "gnn_relabel_workspace_size": (i32, [i64, P(size_t)]),
    "gnn_unique_relabel_noalloc": (i32, [vp, i64, vp, vp, i64, i64, vp, i64, vp, vp, vp, vp, vp]),
    "gnn_feature_store_create": (i32, [vp, i32, i64, i64, i64, i64, vp, P(vp)]),
    "gnn_feature_store_destroy": (i32, [vp]),
    "gnn_feature_store_enable_dynamic": (i32, [vp, P(gnn_dyn_cache_params)]),
    "gnn_dyn_cache_update": (i32, [vp, P(i32), vp, vp]),
    "gnn_dyn_cache_query": (i32, [vp, P(gnn_dyn_cache_info)]),
    "gnn_dyn_cache_state": (i32, [vp, vp, vp, vp]),
    "gnn_host_mapped_pointer": (i32, [vp, P(vp)]),
    "gnn_adjacency_cache_create": (i32, [P(gnn_graph), vp, i64, i64, P(vp), P(i64), P(i64)]),
    "gnn_adjacency_cache_attach": (i32, [vp, P(gnn_graph)]),
    "gnn_adjacency_cache_destroy": (i32, [vp]),
    "gnn_gather_features": (i32, [vp, vp, vp, i64, vp, i64, vp, vp, vp]),
    "gnn_gather_features_match": (i32, [vp, vp, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, vp, vp,
                                        vp, vp]),
    "gnn_batch_overlap": (i32, [P(vp), P(vp), P(i64), i32, vp, vp]),
    "gnn_greedy_order": (i32, [P(i64), i32, i32, P(i32)]),
    "gnn_mean_aggregate": (i32, [vp, vp, i64, vp, i64, vp, i64, i64, i64, vp, i64, vp, vp]),
    "gnn_sage_update": (i32, [vp, vp, i64, vp, i64, i64, i64, vp, i64, vp, vp, i64, i32, vp, i64,
                              vp, vp]),
    "gnn_sage_layer": (i32, [vp, vp, i64, vp, vp, i64, vp, i64, i64, i64, vp, vp, i64, i32, vp, i64,
                             vp, i64, vp, vp]),
    "gnn_minibatch": (i32, [P(gnn_graph), vp, vp, P(i64), i32, P(i32), i32, u64,
                            P(gnn_minibatch_out), vp, size_t, P(gnn_options), vp, vp]),
    "gnn_read_device_status": (i32, [vp, vp, P(i32)]),
    "gnn_timer_create": (i32, [i32, P(vp)]),
    "gnn_timer_destroy": (i32, [vp]),
    "gnn_timer_reset": (i32, [vp]),
    "gnn_timer_elapsed": (i32, [vp, P(i32), P(ctypes.c_float)]),
    # measurement helper (include/gnnmb_probe.h)
    "gnn_copy_probe": (i32, [vp, vp, size_t, vp]),
    "gnn_copy_probe_host": (i32, [vp, vp, size_t, vp]),
    "gnn_hash_probe": (i32, [u64, u64, i64, i64, vp, vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                f"g.build()'` (hipcc, gfx950).  There is no CPU fallback.")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        L.gnn__fastdiv_selfcheck.restype = i64
        L.gnn__fastdiv_selfcheck.argtypes = [u32]
        _lib = L
    return _lib
