"""GNN_FAULT (read once per process, so each case runs in a child process): argument checks come
first, then an injected launch or allocation failure returns GNN_ERR_HIP; nothing touches a
device.  CPU only."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import ctypes, json, sys
sys.path.insert(0, %r)
import graph_mini_pipeline_amd as gm
L = gm.lib()
out = {}
ws = ctypes.c_size_t()
# a relabel with valid (never dereferenced) arguments, then one with an id bound of 0
out["relabel_ok_args"] = L.gnn_unique_relabel(8, 4, 8, None, 4, 100, 8, 8, 8, 8, 8, 8, 1 << 20, None)
out["relabel_bad_args"] = L.gnn_unique_relabel(8, 4, 8, None, 4, 0, 8, 8, 8, 8, 8, 8, 1 << 20, None)
out["noalloc_ok_args"] = L.gnn_unique_relabel_noalloc(8, 4, 8, None, 4, 100, 8, 8, 8, 8, 8, None, None)
# a feature store over a device table: with a cache it allocates, without one it does not
fs = ctypes.c_void_p()
out["store_cache"] = L.gnn_feature_store_create(8, 0, 10, 4, 4, 2, 8, ctypes.byref(fs))
fs2 = ctypes.c_void_p()
out["store_plain"] = L.gnn_feature_store_create(8, 0, 10, 4, 4, 0, None, ctypes.byref(fs2))
L.gnn_feature_store_destroy(fs2)
out["mean_ok_args"] = L.gnn_mean_aggregate(8, 8, 4, None, 2, 8, 4, 4, 4, 8, 4, None, None)
print(json.dumps(out))
''' % ROOT


def _run(fault):
    env = dict(os.environ)
    env.pop("GNN_FAULT", None)
    if fault:
        env["GNN_FAULT"] = fault
    r = subprocess.run([sys.executable, "-c", CHILD], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_launch_fault_after_argument_checks():
    import graph_mini_pipeline_amd as gm
    got = _run("launch")
    assert got["relabel_ok_args"] == gm.GNN_ERR_HIP
    assert got["noalloc_ok_args"] == gm.GNN_ERR_HIP
    assert got["mean_ok_args"] == gm.GNN_ERR_HIP
    assert got["relabel_bad_args"] == gm.GNN_ERR_INVALID_ARG      # checked before the fault
    assert got["store_plain"] == gm.GNN_OK                        # set-up: no launch


def test_alloc_fault_only_where_a_call_allocates():
    import graph_mini_pipeline_amd as gm
    got = _run("alloc")
    assert got["store_cache"] == gm.GNN_ERR_HIP
    assert got["store_plain"] == gm.GNN_OK
    assert got["relabel_bad_args"] == gm.GNN_ERR_INVALID_ARG
