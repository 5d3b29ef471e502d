"""The oracle: a plain, slow, single-threaded CPU reference of the GNN mini-batch path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package.  It never imports the GPU package and shares no code with it; its
arithmetic lives in oracle.c (compiled with gcc) and is driven from here with numpy arrays.

What it computes (GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via
Caching-Sampling-Batching Co-Design, Sec. II.A eq. (1)-(2), Sec. II.B with Fig. 1, Sec. IV.C;
FastGL: A GPU-Efficient Framework for Accelerating Sampling-Based GNN Training at Large Scale, the
sample / ship features / compute iteration):
  for hop l = 1..K with frontier V_{l-1} (V_0 = seeds):
     block l samples min(deg, k_l) neighbours of every frontier node (bottom-k of SplitMix64 keys),
     V_l = ascending unique of V_{l-1} and the sampled ids, with local ids for both lists;
  X = rows of the feature table for V_K;
  h_K = X, and for l = K..1: h_{l-1}[i] = mean of h_l over the sampled neighbours of destination i
  (0 when it has none).
A super-batch of G sub-batches is defined as G independent runs sharing one batch seed.
One GraphSAGE-mean layer over a block (sage_layer; GARDEN Sec. II.A eq. (1)-(2), the model of its
Sec. VI.A): out[i] = relu([h[dst_lid[i]] || mean of h over i's sampled neighbours] @ W + bias),
in double.

The Dynamic-Cache (DynCache; GARDEN Sec. IV.B eq. (5)-(6)): each mini-batch multiplies every
node's score by gamma and adds one per requested row of a node outside the static cache; a refresh,
at the first update call after at least t_update mini-batches, makes the cache the k_dyn nodes of
highest positive score (ties: smaller id); after max_refreshes refreshes (0: no limit) nothing more
is observed or refreshed.

Match and Greedy Reorder (FastGL, "The idea" and "What it costs"): match_positions gives each id's
position in the previous batch's node list (or -1: read from the store); batch_overlap the full
pairwise overlap matrix of a group of batches; greedy_order their nearest-overlap-first order.

Every function here is pinned by the CPU tests (published SplitMix64 outputs, brute force on
hand-built graphs, BFS and dense-matrix special cases, uniformity statistics, exact rationals).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORC_OK = 0
_ERRORS = {-1: "invalid argument", -2: "capacity", -3: "id out of range", -7: "out of memory"}


SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer into `path` (a test
    loads it in place of liboracle.so through GNNMB_ORACLE_LIB, with the ASan runtime preloaded)."""
    subprocess.check_call(["gcc", *SANITIZE_FLAGS, "-std=c11", "-Wall", "-Wextra", "-fPIC",
                           "-shared", "-o", path, _SRC])
    return path


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        alt = os.environ.get("GNNMB_ORACLE_LIB")   # another build of oracle.c (sanitized)
        if not alt:
            build(force=False)
        L = ctypes.CDLL(alt or _LIB)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.orc_mix64.restype = u64
        L.orc_mix64.argtypes = [u64]
        L.orc_splitmix_next.restype = u64
        L.orc_splitmix_next.argtypes = [ctypes.POINTER(u64)]
        L.orc_batch_seed.restype = u64
        L.orc_batch_seed.argtypes = [u64, u64]
        L.orc_hop_seed.restype = u64
        L.orc_hop_seed.argtypes = [u64, i32]
        L.orc_node_seed.restype = u64
        L.orc_node_seed.argtypes = [u64, i32]
        L.orc_edge_key.restype = u64
        L.orc_edge_key.argtypes = [u64, i64]
        L.orc_select_positions.restype = i32
        L.orc_select_positions.argtypes = [u64, i64, i32, vp]
        L.orc_sample_hop.restype = i32
        L.orc_sample_hop.argtypes = [vp, i32, vp, i64, vp, i64, i32, u64, i32, vp, vp, i64,
                                     ctypes.POINTER(i64)]
        L.orc_relabel.restype = i32
        L.orc_relabel.argtypes = [vp, i64, vp, i64, vp, i64, ctypes.POINTER(i64), vp, vp]
        L.orc_gather.restype = i32
        L.orc_gather.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64]
        L.orc_mean.restype = i32
        L.orc_mean.argtypes = [vp, vp, i64, vp, i64, i64, i64, vp, i64]
        L.orc_sage_layer.restype = i32
        L.orc_sage_layer.argtypes = [vp, vp, vp, i64, vp, i64, i64, i64, vp, vp, i64, i32, vp, vp]
        L.orc_dyn_ewma_step.restype = i32
        L.orc_dyn_ewma_step.argtypes = [vp, i64, ctypes.c_double, vp, i64, vp]
        L.orc_dyn_topk.restype = i64
        L.orc_dyn_topk.argtypes = [vp, i64, i64, vp]
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != ORC_OK:
        raise RuntimeError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- hash (SplitMix64 output function; the pages give no generator) ----------------------------

def mix64(z: int) -> int:
    return int(lib().orc_mix64(z & 0xFFFFFFFFFFFFFFFF))


def splitmix_stream(state: int, n: int) -> List[int]:
    s = ctypes.c_uint64(state & 0xFFFFFFFFFFFFFFFF)
    return [int(lib().orc_splitmix_next(ctypes.byref(s))) for _ in range(n)]


def batch_seed(rng_seed: int, b: int) -> int:
    return int(lib().orc_batch_seed(rng_seed & 0xFFFFFFFFFFFFFFFF, b))


def hop_seed(seed64: int, hop: int) -> int:
    return int(lib().orc_hop_seed(seed64 & 0xFFFFFFFFFFFFFFFF, hop))


def node_seed(hs: int, v: int) -> int:
    return int(lib().orc_node_seed(hs & 0xFFFFFFFFFFFFFFFF, v))


def edge_key(ns: int, j: int) -> int:
    return int(lib().orc_edge_key(ns & 0xFFFFFFFFFFFFFFFF, j))


def select_positions(ns: int, deg: int, k: int) -> np.ndarray:
    out = np.zeros(max(1, min(deg, k)), dtype=np.int64)
    _check(lib().orc_select_positions(ns & 0xFFFFFFFFFFFFFFFF, deg, k, _p(out)), "select")
    return out[: min(deg, k)]


# ---- one step at a time ----------------------------------------------------------------------

def _csr(indptr: np.ndarray, indices: np.ndarray):
    indptr = np.ascontiguousarray(indptr)
    assert indptr.dtype in (np.int32, np.int64)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    return indptr, indptr.dtype.itemsize, indices


def sample_hop(indptr: np.ndarray, indices: np.ndarray, frontier: np.ndarray, k: int,
               seed64: int, hop: int):
    """Block of one hop: (blk_indptr int32 [F+1], blk_gid int32 [|E|])."""
    indptr, ib, indices = _csr(indptr, indices)
    frontier = np.ascontiguousarray(frontier, dtype=np.int32)
    n = indptr.shape[0] - 1
    F = frontier.shape[0]
    if F and (frontier.min() < 0 or frontier.max() >= n):
        raise RuntimeError("oracle sample: id out of range")
    deg = (indptr[1:] - indptr[:-1]).astype(np.int64)
    cap = int(np.minimum(deg[frontier], k).sum()) if F else 0
    blk_indptr = np.zeros(F + 1, dtype=np.int32)
    blk_gid = np.zeros(max(cap, 1), dtype=np.int32)
    ne = ctypes.c_int64(0)
    _check(lib().orc_sample_hop(_p(indptr), ib, _p(indices), n, _p(frontier), F, k,
                                seed64 & 0xFFFFFFFFFFFFFFFF, hop, _p(blk_indptr), _p(blk_gid),
                                cap, ctypes.byref(ne)), "sample")
    return blk_indptr, blk_gid[: ne.value]


def relabel(frontier: np.ndarray, gid: np.ndarray):
    """(uniq int32, blk_lid int32 [|gid|], dst_lid int32 [|frontier|])."""
    frontier = np.ascontiguousarray(frontier, dtype=np.int32)
    gid = np.ascontiguousarray(gid, dtype=np.int32)
    F, E = frontier.shape[0], gid.shape[0]
    uniq = np.zeros(F + E + 1, dtype=np.int32)
    blk_lid = np.zeros(E + 1, dtype=np.int32)
    dst_lid = np.zeros(F + 1, dtype=np.int32)
    nu = ctypes.c_int64(0)
    _check(lib().orc_relabel(_p(frontier), F, _p(gid), E, _p(uniq), F + E, ctypes.byref(nu),
                             _p(blk_lid), _p(dst_lid)), "relabel")
    return uniq[: nu.value].copy(), blk_lid[:E].copy(), dst_lid[:F].copy()


def gather(table: np.ndarray, ids: np.ndarray, d: Optional[int] = None) -> np.ndarray:
    """Rows ids of a float32 table (row stride = table.shape[1]); returns [n, d] float32."""
    table = np.ascontiguousarray(table, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    d = table.shape[1] if d is None else d
    out = np.zeros((ids.shape[0], d), dtype=np.float32)
    _check(lib().orc_gather(_p(table), table.shape[1], d, table.shape[0], _p(ids), ids.shape[0],
                            _p(out), d), "gather")
    return out


def mean_aggregate(blk_indptr: np.ndarray, lid: np.ndarray, src: np.ndarray,
                   d: Optional[int] = None) -> np.ndarray:
    """Per-destination mean of src rows; returns [n_dst, d] float32."""
    blk_indptr = np.ascontiguousarray(blk_indptr, dtype=np.int32)
    lid = np.ascontiguousarray(lid, dtype=np.int32)
    src = np.ascontiguousarray(src, dtype=np.float32)
    d = src.shape[1] if d is None else d
    n_dst = blk_indptr.shape[0] - 1
    out = np.zeros((n_dst, d), dtype=np.float32)
    _check(lib().orc_mean(_p(blk_indptr), _p(lid if lid.size else np.zeros(1, np.int32)), n_dst,
                          _p(src if src.size else np.zeros((1, max(d, 1)), np.float32)),
                          src.shape[1] if src.size else d, src.shape[0], d, _p(out), d), "mean")
    return out


def sage_layer(blk_indptr: np.ndarray, lid: np.ndarray, dst_lid: np.ndarray, src: np.ndarray,
               W: np.ndarray, bias: Optional[np.ndarray] = None, relu: bool = True,
               d: Optional[int] = None, with_scale: bool = False):
    """One GraphSAGE-mean layer (GARDEN Sec. II.A eq. (1)-(2)): for destination i,
    a = [src[dst_lid[i]] || mean of src over its sampled neighbours] and
    out[i] = relu(a @ W + bias), W of shape [2d, d_out].  All in double; returns out [n_dst,
    d_out] float64, and with with_scale also sum_k |a_k| |W_kn| + |bias_n| of the same shape."""
    blk_indptr = np.ascontiguousarray(blk_indptr, dtype=np.int32)
    lid = np.ascontiguousarray(lid, dtype=np.int32)
    dst_lid = np.ascontiguousarray(dst_lid, dtype=np.int32)
    src = np.ascontiguousarray(src, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.float32)
    d = src.shape[1] if d is None else d
    if W.shape[0] != 2 * d:
        raise ValueError("W must have 2d rows")
    d_out = W.shape[1]
    n_dst = blk_indptr.shape[0] - 1
    if dst_lid.shape[0] != n_dst:
        raise ValueError("one dst_lid per destination")
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.zeros((n_dst, d_out), dtype=np.float64)
    scale = np.zeros((n_dst, d_out), dtype=np.float64) if with_scale else None
    one_i = np.zeros(1, np.int32)
    _check(lib().orc_sage_layer(_p(blk_indptr), _p(lid if lid.size else one_i),
                                _p(dst_lid if dst_lid.size else one_i), n_dst,
                                _p(src if src.size else np.zeros((1, max(d, 1)), np.float32)),
                                src.shape[1] if src.size else d, src.shape[0], d,
                                _p(W if W.size else np.zeros(1, np.float32)),
                                _p(b) if b is not None else None, d_out, 1 if relu else 0,
                                _p(out if out.size else np.zeros(1)),
                                (_p(scale if scale.size else np.zeros(1)) if with_scale else None)),
           "sage layer")
    return (out, scale) if with_scale else out


# ---- the whole path for one batch ------------------------------------------------------------

@dataclass
class Block:
    indptr: np.ndarray   # int32 [F+1]
    gid: np.ndarray      # int32 [|E|]
    lid: np.ndarray      # int32 [|E|]
    dst_lid: np.ndarray  # int32 [F]
    nodes: np.ndarray    # int32 V_l, ascending unique


@dataclass
class MiniBatch:
    blocks: List[Block]
    x: Optional[np.ndarray] = None          # X = h_K, [|V_K|, d]
    h: List[np.ndarray] = field(default_factory=list)   # h[l] = h_l, l = 0..K-1
    times: Dict[str, float] = field(default_factory=dict)


def sample_khop(indptr, indices, seeds, fanouts: Sequence[int], seed64: int) -> List[Block]:
    seeds = np.ascontiguousarray(seeds, dtype=np.int32)
    if np.unique(seeds).shape[0] != seeds.shape[0]:
        raise RuntimeError("oracle: duplicate seed")
    blocks = []
    front = seeds
    for hop, k in enumerate(fanouts, start=1):
        bi, gid = sample_hop(indptr, indices, front, k, seed64, hop)
        uniq, lid, dst_lid = relabel(front, gid)
        blocks.append(Block(bi, gid, lid, dst_lid, uniq))
        front = uniq
    return blocks


def minibatch(indptr, indices, table: Optional[np.ndarray], seeds, fanouts: Sequence[int],
              seed64: int, d: Optional[int] = None, timed: bool = False) -> MiniBatch:
    """The whole path for one batch; `table` may be None to stop after sampling."""
    t0 = time.perf_counter()
    blocks = sample_khop(indptr, indices, seeds, fanouts, seed64)
    t1 = time.perf_counter()
    mb = MiniBatch(blocks)
    mb.times["sample"] = t1 - t0
    if table is None:
        return mb
    d = table.shape[1] if d is None else d
    mb.x = gather(table, blocks[-1].nodes, d)
    t2 = time.perf_counter()
    K = len(blocks)
    h = [None] * (K + 1)
    h[K] = mb.x
    for l in range(K, 0, -1):
        blk = blocks[l - 1]
        h[l - 1] = mean_aggregate(blk.indptr, blk.lid, h[l], d)
    t3 = time.perf_counter()
    mb.h = h[:K]
    mb.times["gather"] = t2 - t1
    mb.times["aggregate"] = t3 - t2
    return mb


def superbatch(indptr, indices, table, seeds_concat, batch_ptr: Sequence[int],
               fanouts: Sequence[int], seed64: int, d: Optional[int] = None) -> List[MiniBatch]:
    """G sub-batches sharing one batch seed: by definition G independent runs."""
    return [minibatch(indptr, indices, table, seeds_concat[batch_ptr[g]:batch_ptr[g + 1]],
                      fanouts, seed64, d) for g in range(len(batch_ptr) - 1)]


# ---- Dynamic-Cache (GARDEN Sec. IV.B, eq. (5)-(6)) --------------------------------------------

def dyn_ewma_step(score: np.ndarray, gamma: float, ids, is_static: Optional[np.ndarray]) -> None:
    """Eq. (5) for one mini-batch, in place on score (float64 [N])."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    st = None if is_static is None else np.ascontiguousarray(is_static, dtype=np.uint8)
    _check(lib().orc_dyn_ewma_step(_p(score), score.shape[0], float(gamma),
                                   _p(ids) if ids.size else None, ids.size,
                                   _p(st) if st is not None else None), "dyn ewma step")


def dyn_topk(score: np.ndarray, k: int) -> np.ndarray:
    """Eq. (6): ids (ascending) of the k nodes of highest positive score, smaller id on ties."""
    out = np.zeros(max(1, min(k, score.shape[0])), dtype=np.int32)
    c = lib().orc_dyn_topk(_p(score), score.shape[0], int(k), _p(out))
    if c < 0:
        _check(int(c), "dyn topk")
    return out[:c].copy()


class DynCache:
    """The Dynamic-Cache's policy, step by step: observe() is one mini-batch, update() refreshes
    when at least t_update mini-batches were observed since the last refresh."""

    def __init__(self, num_nodes: int, static_ids, gamma: float, k_dyn: int, t_update: int,
                 max_refreshes: int = 0):
        self.score = np.zeros(num_nodes, dtype=np.float64)
        self.is_static = np.zeros(num_nodes, dtype=np.uint8)
        self.is_static[np.asarray(static_ids, dtype=np.int64)] = 1
        self.gamma, self.k_dyn, self.t_update = gamma, k_dyn, t_update
        self.max_refreshes = max_refreshes
        self.steps = 0
        self.since = 0
        self.refreshes = 0
        self.members = np.zeros(0, dtype=np.int32)

    @property
    def frozen(self) -> bool:
        return self.max_refreshes > 0 and self.refreshes >= self.max_refreshes

    def observe(self, ids) -> None:
        if self.frozen:
            return
        dyn_ewma_step(self.score, self.gamma, ids, self.is_static)
        self.steps += 1
        self.since += 1

    def update(self) -> bool:
        if self.frozen or self.since < self.t_update:
            return False
        self.members = dyn_topk(self.score, self.k_dyn)
        self.since = 0
        self.refreshes += 1
        return True


# ---- Match and Greedy Reorder (FastGL: A GPU-Efficient Framework for Accelerating Sampling-Based
# GNN Training at Large Scale, "The idea" and "What it costs") ------------------------------------
#
# Match is result-transparent: a batch's X is gather(table, V_K) whichever rows are copied from the
# previous batch, so its oracle is gather() above; what Match changes is which rows are read from
# the store, namely those of V_K^b outside V_K^{b-1}.

def match_positions(ids, prev_ids) -> np.ndarray:
    """For each id, its position in the previous batch's node list prev_ids, or -1 (a row read from
    the store).  Written as the definition: a dictionary of prev_ids' positions."""
    where = {int(v): p for p, v in enumerate(np.asarray(prev_ids).tolist())}
    return np.array([where.get(int(v), -1) for v in np.asarray(ids).tolist()], dtype=np.int32)


def batch_overlap(lists) -> np.ndarray:
    """The group's full pairwise overlap matrix: entry (a, b) = |L_a ∩ L_b| (|L_a| on the diagonal)."""
    B = len(lists)
    sets = [set(np.asarray(l).tolist()) for l in lists]
    m = np.zeros((B, B), dtype=np.int64)
    for a in range(B):
        for b in range(B):
            m[a, b] = len(sets[a] & sets[b])
    return m


def greedy_order(overlap, first: int = 0) -> List[int]:
    """Nearest-overlap-first: start with batch `first`; each next batch is the one not yet placed
    that shares the most nodes with the last placed (ties: the smaller index)."""
    m = np.asarray(overlap)
    B = m.shape[0]
    order = [first]
    left = [b for b in range(B) if b != first]
    while left:
        last = order[-1]
        best = left[0]
        for b in left[1:]:
            if m[last, b] > m[last, best]:
                best = b
        order.append(best)
        left.remove(best)
    return order
