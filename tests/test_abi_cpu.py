"""The C-ABI library on the CPU: it loads, exports every function include/gnnmb.h declares, its
ctypes mirror matches the C layout, and host-side logic (capacities, workspace sizes, argument
validation, the invariant-divisor division) behaves.  No call here launches GPU work: every call
either is pure host arithmetic or fails validation before touching the device."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import graph_mini_pipeline_amd as gm
from graph_mini_pipeline_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gnnmb.h", "gnnmb_probe.h")]


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gnn_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 17
    L = gm.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in _abi.SIGNATURES, f"{n} has no ctypes signature"


def test_ctypes_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stddef.h>
#include <stdio.h>
#include "gnnmb.h"
#define S(T) printf(#T " %zu\n", sizeof(T));
#define O(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  S(gnn_graph) S(gnn_caps) S(gnn_block) S(gnn_blocks) S(gnn_options) S(gnn_minibatch_out)
  S(gnn_dyn_cache_params) S(gnn_dyn_cache_info)
  O(gnn_graph, indices) O(gnn_graph, adj_rows) O(gnn_caps, nodes) O(gnn_blocks, counts) O(gnn_minibatch_out, ld_h)
  O(gnn_minibatch_out, x) O(gnn_options, flags) O(gnn_options, d_hits) O(gnn_dyn_cache_params, flags)
  O(gnn_dyn_cache_info, members) O(gnn_dyn_cache_info, last_evicted) return 0; }
''')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                           str(exe)])
    got = dict(line.rsplit(" ", 1) for line in subprocess.check_output([str(exe)]).decode().split("\n") if line)
    py = {
        "gnn_graph": ctypes.sizeof(_abi.gnn_graph), "gnn_caps": ctypes.sizeof(_abi.gnn_caps),
        "gnn_block": ctypes.sizeof(_abi.gnn_block), "gnn_blocks": ctypes.sizeof(_abi.gnn_blocks),
        "gnn_options": ctypes.sizeof(_abi.gnn_options),
        "gnn_minibatch_out": ctypes.sizeof(_abi.gnn_minibatch_out),
        "gnn_graph.indices": _abi.gnn_graph.indices.offset,
        "gnn_graph.adj_rows": _abi.gnn_graph.adj_rows.offset,
        "gnn_caps.nodes": _abi.gnn_caps.nodes.offset,
        "gnn_blocks.counts": _abi.gnn_blocks.counts.offset,
        "gnn_minibatch_out.ld_h": _abi.gnn_minibatch_out.ld_h.offset,
        "gnn_minibatch_out.x": _abi.gnn_minibatch_out.x.offset,
        "gnn_options.flags": _abi.gnn_options.flags.offset,
        "gnn_options.d_hits": _abi.gnn_options.d_hits.offset,
        "gnn_dyn_cache_params": ctypes.sizeof(_abi.gnn_dyn_cache_params),
        "gnn_dyn_cache_info": ctypes.sizeof(_abi.gnn_dyn_cache_info),
        "gnn_dyn_cache_params.flags": _abi.gnn_dyn_cache_params.flags.offset,
        "gnn_dyn_cache_info.members": _abi.gnn_dyn_cache_info.members.offset,
        "gnn_dyn_cache_info.last_evicted": _abi.gnn_dyn_cache_info.last_evicted.offset,
    }
    for k, v in py.items():
        assert int(got[k]) == v, k


def test_capacity_chain():
    caps = gm.gnn_capacity(1024, [15, 10, 5], 111_000_000)
    assert caps.num_hops == 3 and caps.n_seeds == 1024
    assert list(caps.frontier[:3]) == [1024, 16384, 180224]
    assert list(caps.edges[:3]) == [15360, 163840, 901120]
    assert list(caps.nodes[:3]) == [16384, 180224, 1081344]
    caps = gm.gnn_capacity(256, [10, 5], 10_000)      # the N cap applies
    assert list(caps.nodes[:2]) == [2816, 10000] and caps.frontier[1] == 2816
    caps = gm.gnn_capacity(0, [3], 5)
    assert caps.edges[0] == 0 and caps.nodes[0] == 0


@pytest.mark.parametrize("bad", [dict(fanouts=[]), dict(fanouts=[0]), dict(fanouts=[-1, 2]),
                                 dict(n=-1), dict(N=0), dict(fanouts=[1] * 9)])
def test_capacity_rejects(bad):
    with pytest.raises(gm.GnnError) as e:
        gm.gnn_capacity(bad.get("n", 4), bad.get("fanouts", [2]), bad.get("N", 10))
    assert e.value.status == gm.GNN_ERR_INVALID_ARG


def test_capacity_unsupported_sizes():
    gm.gnn_capacity(4, [832], 10)               # the largest fanout: a quarter of the LDS class
    for f in (833, 5000):
        with pytest.raises(gm.GnnError) as e:
            gm.gnn_capacity(4, [f], 10)         # fanout above the largest LDS class
        assert e.value.status == gm.GNN_ERR_UNSUPPORTED
    with pytest.raises(gm.GnnError) as e:
        gm.gnn_capacity(2**30, [4], 2**31 - 1)  # edges overflow int32
    assert e.value.status == gm.GNN_ERR_UNSUPPORTED


def test_workspace_grows_with_graph():
    caps = gm.gnn_capacity(1024, [25, 10], 233_000)
    a = gm.gnn_workspace_size(caps, 233_000)
    b = gm.gnn_workspace_size(caps, 250_000_000)
    assert 0 < a < b
    assert b >= 2 * (250_000_000 // 32) * 4    # bitmap + word prefixes
    assert gm.gnn_relabel_workspace_size(1000) > 0


def test_status_strings():
    for s in range(-6, 1):
        assert gm.gnn_status_string(s)


def test_batch_seed_is_splitmix_stream():
    import oracle
    for r in (0, 1234567):
        for b in range(5):
            assert gm.gnn_batch_seed(r, b) == oracle.batch_seed(r, b)
    seed, expected = __import__("tests.helpers", fromlist=["x"]).read_golden_splitmix()
    assert [gm.gnn_batch_seed(seed, b) for b in range(5)] == expected


def test_fastdiv_selfcheck():
    assert gm.lib().gnn__fastdiv_selfcheck(5000) == 0


def test_validation_before_device_work():
    L = gm.lib()
    caps = gm.gnn_capacity(4, [2], 10)
    blocks = _abi.gnn_blocks()
    blocks.caps = caps
    fo = (ctypes.c_int32 * 1)(2)
    # no graph
    assert L.gnn_sample_khop(None, None, 4, fo, 1, 0, ctypes.byref(blocks), None, 0, None,
                             None) == gm.GNN_ERR_INVALID_ARG
    g = _abi.gnn_graph()
    g.num_nodes, g.num_edges, g.indptr, g.indptr_bytes, g.indices = 10, 5, 8, 2, 8
    assert L.gnn_sample_khop(ctypes.byref(g), 8, 4, fo, 1, 0, ctypes.byref(blocks), 8, 1 << 20,
                             None, None) == gm.GNN_ERR_INVALID_ARG   # indptr width 2
    g.indptr_bytes = 4
    # blocks without counts / arrays
    assert L.gnn_sample_khop(ctypes.byref(g), 8, 4, fo, 1, 0, ctypes.byref(blocks), 8, 1 << 20,
                             None, None) == gm.GNN_ERR_INVALID_ARG
    # options: wave bound below group bound
    o = _abi.gnn_options()
    o.group_max_deg, o.wave_max_deg = 100, 10
    blocks.counts = 8
    h = blocks.hop[0]
    h.indptr = h.gid = h.lid = h.dst_lid = h.nodes = 8
    assert L.gnn_sample_khop(ctypes.byref(g), 8, 4, fo, 1, 0, ctypes.byref(blocks), 8, 1 << 20,
                             ctypes.byref(o), None) == gm.GNN_ERR_INVALID_ARG
    # workspace too small
    assert L.gnn_sample_khop(ctypes.byref(g), 8, 4, fo, 1, 0, ctypes.byref(blocks), 8, 16,
                             None, None) == gm.GNN_ERR_CAPACITY
    # seeds count differs from the caps
    assert L.gnn_sample_khop(ctypes.byref(g), 8, 3, fo, 1, 0, ctypes.byref(blocks), 8, 1 << 20,
                             None, None) == gm.GNN_ERR_INVALID_ARG
    # mean: ld below d
    assert L.gnn_mean_aggregate(8, 8, 4, None, 2, 8, 3, 4, 4, 8, 4, None,
                                None) == gm.GNN_ERR_INVALID_ARG
    # sage layer (each call differs from a well-formed one in one argument): d_out 0, ld_out
    # below d_out, ld_agg below d, missing W
    args = [8, 8, 4, 8, None, 2, 8, 4, 4, 4, 8, None, 4, 1, 8, 4, 8, 4, None, None]
    for i, v in ((12, 0), (17, 3), (15, 3), (10, None)):
        bad = list(args)
        bad[i] = v
        assert L.gnn_sage_layer(*bad) == gm.GNN_ERR_INVALID_ARG, i
    uargs = [8, None, 2, 8, 4, 4, 4, 8, 4, 8, None, 4, 1, 8, 4, None, None]
    for i, v in ((11, 0), (14, 3), (8, 3), (9, None), (0, None)):
        bad = list(uargs)
        bad[i] = v
        assert L.gnn_sage_update(*bad) == gm.GNN_ERR_INVALID_ARG, i
    # relabel: id bound 0
    n = ctypes.c_size_t()
    assert L.gnn_relabel_workspace_size(0, ctypes.byref(n)) == gm.GNN_ERR_INVALID_ARG
    # timer: zero records
    t = ctypes.c_void_p()
    assert L.gnn_timer_create(0, ctypes.byref(t)) == gm.GNN_ERR_INVALID_ARG
    # feature store: ld < d
    assert L.gnn_feature_store_create(8, 0, 10, 8, 4, 0, None,
                                      ctypes.byref(t)) == gm.GNN_ERR_INVALID_ARG
    # adjacency cache: no handle out, more hot ids than nodes, negative budget, missing hot
    # order, a graph with only one of its two cache pointers; mapping a NULL host pointer
    g.indptr_bytes = 4
    assert L.gnn_adjacency_cache_create(ctypes.byref(g), 8, 1, 10, None, None,
                                        None) == gm.GNN_ERR_INVALID_ARG
    assert L.gnn_adjacency_cache_create(ctypes.byref(g), 8, 11, 10, ctypes.byref(t), None,
                                        None) == gm.GNN_ERR_INVALID_ARG
    assert L.gnn_adjacency_cache_create(ctypes.byref(g), 8, 1, -1, ctypes.byref(t), None,
                                        None) == gm.GNN_ERR_INVALID_ARG
    assert L.gnn_adjacency_cache_create(ctypes.byref(g), None, 1, 10, ctypes.byref(t), None,
                                        None) == gm.GNN_ERR_INVALID_ARG
    g.adj_off = 8
    assert L.gnn_adjacency_cache_create(ctypes.byref(g), 8, 1, 10, ctypes.byref(t), None,
                                        None) == gm.GNN_ERR_INVALID_ARG
    assert L.gnn_sample_khop(ctypes.byref(g), 8, 4, fo, 1, 0, ctypes.byref(blocks), 8, 1 << 20,
                             None, None) == gm.GNN_ERR_INVALID_ARG
    g.adj_off = None
    assert L.gnn_adjacency_cache_attach(None, None) == gm.GNN_ERR_INVALID_ARG
    assert L.gnn_adjacency_cache_attach(None, ctypes.byref(g)) == gm.GNN_OK   # detach
    assert L.gnn_adjacency_cache_destroy(None) == gm.GNN_OK
    p = ctypes.c_void_p()
    assert L.gnn_host_mapped_pointer(None, ctypes.byref(p)) == gm.GNN_ERR_INVALID_ARG


def test_header_constants_match_binding():
    import re
    text = open(os.path.join(ROOT, "include", "gnnmb.h")).read()
    consts = {m.group(1): int(m.group(2)) for m in
              re.finditer(r"#define\s+(GNN_[A-Z0-9_]+)\s+\(?(-?\d+)u?\)?", text)}
    assert consts, "no constants found"
    for name, value in consts.items():
        assert getattr(_abi, name) == value, name


def test_superbatch_union_block_must_fit_int32():
    """Each sub-batch's caps fit int32, but the union block of 16 of them would not: the call is
    rejected on the host (GNN_ERR_UNSUPPORTED) before any device work; 2 sub-batches fit."""
    L = gm.lib()
    N = 2**31 - 1
    fan = [800]
    fo = (ctypes.c_int32 * 1)(*fan)
    caps = gm.gnn_capacity(2**20, fan, N)
    assert caps.edges[0] == 2**20 * 800 < 2**31
    g = _abi.gnn_graph()
    g.num_nodes, g.num_edges, g.indptr, g.indptr_bytes, g.indices = N, 5, 8, 8, 8
    fs = ctypes.c_void_p()
    # a store over a (never read) device table: no cache, so creation touches no device
    assert L.gnn_feature_store_create(8, 0, N, 1, 1, 0, None, ctypes.byref(fs)) == gm.GNN_OK

    def outs(G):
        arr = (_abi.gnn_minibatch_out * G)()
        for m in arr:
            m.blocks.caps = caps
            m.blocks.counts = 8
            h = m.blocks.hop[0]
            h.indptr = h.gid = h.lid = h.dst_lid = h.nodes = 8
            m.x = 8
            m.h[0] = 8
            m.ld_h = 1     # d = 1: rows * d stays within the flat index bound
        return arr

    try:
        for G, want in ((16, gm.GNN_ERR_UNSUPPORTED), (2, gm.GNN_ERR_CAPACITY)):
            ptr = (ctypes.c_int64 * (G + 1))(*[i * 2**20 for i in range(G + 1)])
            # with a workspace of 16 bytes: the fitting super-batch stops at the workspace check
            st = L.gnn_minibatch(ctypes.byref(g), fs, 8, ptr, G, fo, 1, 0, outs(G), 8, 16, None,
                                 None, None)
            assert st == want, (G, st)
    finally:
        L.gnn_feature_store_destroy(fs)


def test_noalloc_relabel_host_checks():
    """The allocation-free relabel's scratch covers its largest id range, and sizes beyond it are
    refused on the host before any device work."""
    need = gm.gnn_relabel_workspace_size(gm.GNN_NOALLOC_MAX_IDS)
    assert need <= gm.GNN_NOALLOC_SCRATCH_BYTES
    assert gm.gnn_relabel_workspace_size(2 * gm.GNN_NOALLOC_MAX_IDS) > gm.GNN_NOALLOC_SCRATCH_BYTES
    L = gm.lib()
    # id bound above the scratch's maximum
    assert L.gnn_unique_relabel_noalloc(8, 4, 8, None, 4, gm.GNN_NOALLOC_MAX_IDS + 1, 8, 8, 8, 8,
                                        8, None, None) == gm.GNN_ERR_UNSUPPORTED
    # the argument checks of gnn_unique_relabel: missing count output, id bound 0
    assert L.gnn_unique_relabel_noalloc(8, 4, 8, None, 4, 100, 8, 8, None, 8, 8, None,
                                        None) == gm.GNN_ERR_INVALID_ARG
    assert L.gnn_unique_relabel_noalloc(8, 4, 8, None, 4, 0, 8, 8, 8, 8, 8, None,
                                        None) == gm.GNN_ERR_INVALID_ARG


def test_relabel_path_flags_exclusive():
    o = gm.Options(relabel="sort")
    o.c()
    with pytest.raises(ValueError):
        gm.Options(relabel="hash").c()
    L = gm.lib()
    caps = gm.gnn_capacity(4, [2], 10)
    blocks = _abi.gnn_blocks()
    blocks.caps = caps
    blocks.counts = 8
    h = blocks.hop[0]
    h.indptr = h.gid = h.lid = h.dst_lid = h.nodes = 8
    g = _abi.gnn_graph()
    g.num_nodes, g.num_edges, g.indptr, g.indptr_bytes, g.indices = 10, 5, 8, 4, 8
    fo = (ctypes.c_int32 * 1)(2)
    both = _abi.gnn_options()
    both.flags = gm.GNN_RELABEL_SORT | gm.GNN_RELABEL_BITMAP
    assert L.gnn_sample_khop(ctypes.byref(g), 8, 4, fo, 1, 0, ctypes.byref(blocks), 8, 1 << 20,
                             ctypes.byref(both), None) == gm.GNN_ERR_INVALID_ARG


def test_dynamic_cache_host_checks():
    """The Dynamic-Cache entry points refuse a missing store or parameters before any device work."""
    L = gm.lib()
    p = _abi.gnn_dyn_cache_params(0.9, 10, 2, 0, 0)
    assert L.gnn_feature_store_enable_dynamic(None, ctypes.byref(p)) == gm.GNN_ERR_INVALID_ARG
    assert L.gnn_feature_store_enable_dynamic(8, None) == gm.GNN_ERR_INVALID_ARG
    r = ctypes.c_int32(7)
    assert L.gnn_dyn_cache_update(None, ctypes.byref(r), None, None) == gm.GNN_ERR_INVALID_ARG
    assert r.value == 0
    info = _abi.gnn_dyn_cache_info()
    assert L.gnn_dyn_cache_query(None, ctypes.byref(info)) == gm.GNN_ERR_INVALID_ARG
    assert L.gnn_dyn_cache_state(None, None, None, None) == gm.GNN_ERR_INVALID_ARG
