"""Seeded synthetic inputs: R-MAT graphs in CSR-by-destination form, seed orders and feature tables.

This module is the only code shared by the oracle side and the GPU side, and it holds none of the
mini-batch method's arithmetic (no sampling hash, no relabel, no gather, no mean).  Its random
stream is MurmurHash3's 32-bit finalizer (Appleby) applied to a counter, which is unrelated to the
64-bit sampling hash of the method.

Everything is written with torch tensor ops so that the same code runs on the CPU (small graphs,
tests) and on a GPU (billion-edge graphs, where host-side generation would take too long).  All
operations are integer ops, sorts and uniques, so a graph is the same on either device; the float
feature fill may differ in the last ulp between devices, which never matters because both sides of
any comparison read the one buffer that was filled.

Graph recipe (stated in full so that it can be re-implemented):
  * R-MAT (Chakrabarti, Zhan, Faloutsos 2004) on 2^L ids, L = ceil(log2 N).  Draw i, level l uses a
    16-bit uniform u taken from word u32(gseed, i*ceil(L/2) + l//2), half (l % 2).  Quadrants, in the
    order a|b|c|d on the 65536 scale: row (source) bit = [u in c or d], column (destination) bit =
    [u in b or d]; bits are filled most significant first.
  * A draw is rejected if an endpoint is >= N or it is a self-loop.  The graph keeps the first E
    distinct (source, destination) pairs in draw order.
  * A seeded permutation scrambles node ids (so hubs are not the smallest ids).
  * CSR by destination: row v lists the sources of edges (u, v), ascending.
"""
from __future__ import annotations

import ctypes
import math
import os
import shutil
import subprocess
from dataclasses import dataclass, field
from typing import List, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "csrc", "rmat.hip")

__all__ = [
    "u32", "Graph", "rmat_csr", "node_order", "fill_features", "CONFIGS", "WorkloadConfig",
    "build_graph", "make_features", "epoch_seed_order", "batch_seeds",
]

_M32 = 0xFFFFFFFF


def _mul32(h: torch.Tensor, c: int) -> torch.Tensor:
    """(h * c) mod 2^32 for h in [0, 2^32), without int64 overflow: split c into 16-bit halves."""
    lo = c & 0xFFFF
    hi = (c >> 16) & 0xFFFF
    return ((h * lo) + (((h * hi) & 0xFFFF) << 16)) & _M32


def _fmix32(h: torch.Tensor) -> torch.Tensor:
    """MurmurHash3 32-bit finalizer (Appleby), on int64 tensors holding values in [0, 2^32)."""
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def u32(seed: int, ctr: torch.Tensor) -> torch.Tensor:
    """Counter-based 32-bit uniform word: int64 tensor in [0, 2^32) for int64 counters ctr >= 0."""
    s0 = seed & _M32
    s1 = (seed >> 32) & _M32
    a = ctr & _M32
    b = ctr >> 32
    h = _fmix32(a ^ s0)
    h = _fmix32(((h + _mul32(b, 0x9E3779B1)) & _M32) ^ s1)
    return h


def sub_seed(rng_seed: int, tag: int) -> int:
    """A 64-bit sub-seed for stream `tag` of a workload seed (tags: 1 graph, 2 scramble, 3 seeds,
    4 features, 5 epoch order, 6 pre-sampling)."""
    w = u32(rng_seed, torch.tensor([2 * tag, 2 * tag + 1], dtype=torch.int64))
    return int(w[0]) << 32 | int(w[1])


@dataclass
class Graph:
    """CSR by destination.  indptr: int32 or int64 [N+1]; indices: int32 [E]."""
    num_nodes: int
    indptr: torch.Tensor
    indices: torch.Tensor

    @property
    def num_edges(self) -> int:
        return int(self.indices.numel())

    def degrees(self) -> torch.Tensor:
        return (self.indptr[1:] - self.indptr[:-1]).to(torch.int64)

    def to(self, device) -> "Graph":
        return Graph(self.num_nodes, self.indptr.to(device), self.indices.to(device))


def rmat_csr(num_nodes: int, num_edges: int, a: float, b: float, c: float, seed: int,
             indptr_dtype=torch.int32, device="cpu", max_chunk: int = 1 << 27) -> Graph:
    """Seeded R-MAT graph with exactly `num_edges` distinct non-loop edges, CSR by destination."""
    n = int(num_nodes)
    assert n >= 2 and num_edges <= n * (n - 1)
    dev = torch.device(device)
    L = max(1, math.ceil(math.log2(n)))
    W = (L + 1) // 2
    ta = round(a * 65536)
    tb = round((a + b) * 65536)
    tc = round((a + b + c) * 65536)
    gseed = sub_seed(seed, 1)
    accepted = torch.empty(0, dtype=torch.int64, device=dev)  # sorted unique keys dst*n+src
    counter = 0
    while accepted.numel() < num_edges:
        need = num_edges - accepted.numel()
        m = min(max_chunk, int(need * 1.3) + 4096)
        idx = torch.arange(counter, counter + m, dtype=torch.int64, device=dev)
        counter += m
        src = torch.zeros(m, dtype=torch.int64, device=dev)
        dst = torch.zeros(m, dtype=torch.int64, device=dev)
        word = None
        for lvl in range(L):
            if lvl % 2 == 0:
                word = u32(gseed, idx * W + lvl // 2)
            u = (word >> (16 * (lvl % 2))) & 0xFFFF
            sbit = (u >= tb).to(torch.int64)
            dbit = (((u >= ta) & (u < tb)) | (u >= tc)).to(torch.int64)
            src = src * 2 + sbit
            dst = dst * 2 + dbit
        del word, u
        ok = (src < n) & (dst < n) & (src != dst)
        key = (dst * n + src)[ok]
        pos = idx[ok]
        del src, dst, ok, idx
        uk, inv = torch.unique(key, sorted=True, return_inverse=True)
        first = torch.full((uk.numel(),), torch.iinfo(torch.int64).max, dtype=torch.int64, device=dev)
        first.scatter_reduce_(0, inv, pos, reduce="amin")
        del inv, key, pos
        if accepted.numel():
            at = torch.searchsorted(accepted, uk).clamp_(max=accepted.numel() - 1)
            fresh = accepted[at] != uk
            uk, first = uk[fresh], first[fresh]
            del at, fresh
        order = torch.argsort(first)[:need]
        accepted = torch.sort(torch.cat([accepted, uk[order]])).values
        del uk, first, order
    dst = accepted // n
    src = accepted - dst * n
    del accepted
    new_id = _scramble(n, sub_seed(seed, 2), dev)
    dst = new_id[dst]
    src = new_id[src]
    key = torch.sort(dst * n + src).values
    del dst, src
    dst = key // n
    indices = (key - dst * n).to(torch.int32)
    del key
    deg = torch.bincount(dst, minlength=n)
    del dst
    indptr = torch.zeros(n + 1, dtype=torch.int64, device=dev)
    indptr[1:] = torch.cumsum(deg, 0)
    return Graph(n, indptr.to(indptr_dtype), indices)


def build() -> str:
    """Compile the R-MAT draw kernel (csrc/rmat.hip) into libsynth.so for gfx950."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", _SRC, "-o", tmp],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, _LIB)
    return _LIB


_synth_lib = None


def _draw_lib():
    global _synth_lib
    if _synth_lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is missing: run synth.build()")
        L = ctypes.CDLL(_LIB)
        i64, u64, i32, u32, vp = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32,
                                  ctypes.c_void_p)
        L.synth_rmat_draw.restype = ctypes.c_int
        L.synth_rmat_draw.argtypes = [u64, i64, i64, i32, u32, u32, u32, i64, vp, i64, i64, vp, vp,
                                      vp, i64, vp]
        _synth_lib = L
    return _synth_lib


def rmat_csr_partitioned(num_nodes: int, num_edges: int, a: float, b: float, c: float, seed: int,
                         indptr_dtype=torch.int64, device="cuda", draws_per_part: int = 1 << 28,
                         draws: Optional[int] = None) -> Graph:
    """The same graph as rmat_csr, built on a GPU for billions of edges.

    The draws are regenerated by a HIP kernel once per range of (scrambled) destination ids;
    each range keeps its distinct pairs with their first draw index; a histogram of those indices
    finds the cut that keeps exactly the first num_edges distinct pairs in draw order.  Ranges are
    in destination order and each is sorted, so concatenating them gives the CSR by destination."""
    n = int(num_nodes)
    dev = torch.device(device)
    assert dev.type == "cuda"
    L = max(1, math.ceil(math.log2(n)))
    ta, tb, tc = round(a * 65536), round((a + b) * 65536), round((a + b + c) * 65536)
    gseed = sub_seed(seed, 1)
    new_id = _scramble(n, sub_seed(seed, 2), dev).contiguous()
    lib = _draw_lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    D = int(draws) if draws else int(num_edges * 1.06) + (1 << 20)
    while True:
        parts = max(1, -(-D // draws_per_part))
        cap = int(D / parts * 1.25) + (1 << 20)
        keys = torch.empty(cap, dtype=torch.int64, device=dev)
        idx = torch.empty(cap, dtype=torch.int64, device=dev)
        cnt = torch.zeros(1, dtype=torch.int64, device=dev)
        per_part = []
        for p in range(parts):
            lo, hi = p * n // parts, (p + 1) * n // parts
            cnt.zero_()
            rc = lib.synth_rmat_draw(gseed, 0, D, L, ta, tb, tc, n, new_id.data_ptr(), lo, hi,
                                     keys.data_ptr(), idx.data_ptr(), cnt.data_ptr(), cap, stream)
            if rc != 0:
                raise RuntimeError(f"synth_rmat_draw failed ({rc})")
            m = int(cnt.item())
            if m > cap:
                raise RuntimeError("draw buffer too small for a partition")
            uk, inv = torch.unique(keys[:m], sorted=True, return_inverse=True)
            first = torch.full((uk.numel(),), torch.iinfo(torch.int64).max, dtype=torch.int64, device=dev)
            first.scatter_reduce_(0, inv, idx[:m], reduce="amin")
            del inv
            per_part.append((uk, first))
        del keys, idx
        total = sum(u.numel() for u, _ in per_part)
        if total >= num_edges:
            break
        del per_part
        D = int(D * 1.25) + (1 << 20)
    # cut: the num_edges-th smallest first-draw index over all ranges
    shift = max(0, (D - 1).bit_length() - 22)
    nb = (D >> shift) + 1
    hist = torch.zeros(nb, dtype=torch.int64, device=dev)
    for _, f in per_part:
        hist += torch.bincount(f >> shift, minlength=nb)
    cum = torch.cumsum(hist, 0)
    bstar = int(torch.searchsorted(cum, torch.tensor([num_edges], device=dev)).item())
    before = int(cum[bstar - 1].item()) if bstar > 0 else 0
    vals = torch.sort(torch.cat([f[(f >> shift) == bstar] for _, f in per_part])).values
    t_star = int(vals[num_edges - before - 1].item())
    indices, deg = [], torch.zeros(n, dtype=torch.int64, device=dev)
    for uk, f in per_part:
        kept = uk[f <= t_star]
        dst = kept // n
        deg += torch.bincount(dst, minlength=n)
        indices.append((kept - dst * n).to(torch.int32))
        del kept, dst
    del per_part
    indices = torch.cat(indices)
    assert indices.numel() == num_edges
    indptr = torch.zeros(n + 1, dtype=torch.int64, device=dev)
    indptr[1:] = torch.cumsum(deg, 0)
    return Graph(n, indptr.to(indptr_dtype), indices)


def _scramble(n: int, seed: int, dev) -> torch.Tensor:
    """Bijection [0,n) -> [0,n): new_id[v] = rank of (u32(seed, v), v)."""
    v = torch.arange(n, dtype=torch.int64, device=dev)
    order = torch.argsort(u32(seed, v) * (1 << 31) + v)
    new_id = torch.empty(n, dtype=torch.int64, device=dev)
    new_id[order] = v
    return new_id


def node_order(n: int, seed: int, device="cpu") -> torch.Tensor:
    """A seeded order of all node ids (int64): ids sorted by (u32(seed, v), v)."""
    v = torch.arange(n, dtype=torch.int64, device=device)
    return torch.argsort(u32(seed, v) * (1 << 31) + v)


def fill_features(out: torch.Tensor, d: int, dist: str, seed: int, row0: int = 0,
                  rows_per_chunk: Optional[int] = None) -> None:
    """Fill out[:, :d] (float32, any row stride >= d) with seeded values; padding columns get 0.

    Element (r, t) of the full table uses counter r*d + t.  'uniform': U[-1,1] from the top 24
    bits of one word.  'normal': Box-Muller, z = sqrt(-2 ln u1) cos(2 pi u2) in double, with
    u1, u2 from words 2e and 2e+1 (each (w + 0.5) / 2^32)."""
    rows = out.shape[0]
    dev = out.device
    if rows_per_chunk is None:
        rows_per_chunk = max(1, (1 << 25) // d) if dev.type == "cuda" else 1 << 16
    if out.shape[1] > d:
        out[:, d:] = 0
    for r0 in range(0, rows, rows_per_chunk):
        r1 = min(rows, r0 + rows_per_chunk)
        e = (torch.arange(r0 + row0, r1 + row0, dtype=torch.int64, device=dev)[:, None] * d
             + torch.arange(d, dtype=torch.int64, device=dev)[None, :])
        if dist == "uniform":
            w = u32(seed, e)
            val = ((w >> 8).to(torch.float64) + 0.5) / float(1 << 24) * 2.0 - 1.0
        elif dist == "normal":
            u1 = (u32(seed, 2 * e).to(torch.float64) + 0.5) / 4294967296.0
            u2 = (u32(seed, 2 * e + 1).to(torch.float64) + 0.5) / 4294967296.0
            val = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)
        else:
            raise ValueError(dist)
        out[r0:r1, :d] = val.to(torch.float32)


@dataclass
class WorkloadConfig:
    """One synthetic workload, named by what it is."""
    name: str
    num_nodes: int
    num_edges: int
    indptr_bytes: int
    d: int
    dist: str
    batch: int
    fanouts: List[int]
    rng_seed: int = 0
    rmat: tuple = (0.57, 0.19, 0.19)
    n_train: Optional[int] = None      # training seeds per epoch (None: whole batches from the order)
    group: int = 1                     # sub-batches per super-batch
    ld_pad: int = 4                    # device feature row stride is d rounded up to this
    host_features: bool = False        # feature table in pinned host memory
    cache_bytes: int = 0               # HBM hot-row cache budget
    notes: str = ""

    @property
    def ld(self) -> int:
        p = self.ld_pad
        return (self.d + p - 1) // p * p


CONFIGS = {
    "tiny": WorkloadConfig(
        "tiny", 10_000, 160_000, 4, 64, "uniform", 256, [10, 5], notes="correctness case"),
    "dense": WorkloadConfig(
        "dense", 233_000, 115_000_000, 4, 602, "normal", 1024, [25, 10], n_train=150_000,
        notes="dense neighbourhoods, shaped like a 0.2M-node / 114M-edge / 602-d social graph"),
    "mid": WorkloadConfig(
        "mid", 2_450_000, 124_000_000, 4, 100, "normal", 1024, [15, 10, 5], group=8,
        notes="mid-scale, shaped like a 2.4M-node / 124M-directed-edge / 100-d product graph"),
    "large": WorkloadConfig(
        "large", 111_000_000, 1_600_000_000, 8, 128, "normal", 1024, [15, 10, 5],
        notes="large in-HBM, shaped like a 111M-node / 1.6B-edge / 128-d citation graph"),
    # 64-d rather than 128-d: a process can pin about 67 GiB of host memory on the measuring box
    # (hipHostMalloc fails beyond ~71 GB), so the host table is 64 GB; the cache keeps the same
    # 67.1M rows (26.8% of the nodes) at 16 GiB.
    "billion": WorkloadConfig(
        "billion", 250_000_000, 4_000_000_000, 8, 64, "normal", 4096, [15, 10, 5],
        host_features=True, cache_bytes=16 << 30,
        notes="billion-edge, 64-d features in pinned host memory (64 GB) with a 16 GiB HBM "
              "hot-row cache (26.8% of rows)"),
}


# Above this many edges a GPU build regenerates draws per destination range (rmat_csr_partitioned)
# instead of holding every draw in memory at once; both give the same graph.
PARTITIONED_EDGES = 1 << 28


def build_graph(cfg: WorkloadConfig, device="cpu") -> Graph:
    dt = torch.int32 if cfg.indptr_bytes == 4 else torch.int64
    a, b, c = cfg.rmat
    if torch.device(device).type == "cuda" and cfg.num_edges >= PARTITIONED_EDGES:
        return rmat_csr_partitioned(cfg.num_nodes, cfg.num_edges, a, b, c, cfg.rng_seed, dt, device)
    return rmat_csr(cfg.num_nodes, cfg.num_edges, a, b, c, cfg.rng_seed, dt, device)


def make_features(cfg: WorkloadConfig, out: torch.Tensor, device=None,
                  staging_rows: int = 1 << 21) -> None:
    """Fill the feature table out[N, ld].  A host table with a GPU `device` given is filled through
    a device staging buffer, chunk by chunk (the same values: every element has its own counter)."""
    seed = sub_seed(cfg.rng_seed, 4)
    if out.is_cuda or device is None:
        fill_features(out, cfg.d, cfg.dist, seed)
        return
    stage = torch.empty(min(staging_rows, out.shape[0]), out.shape[1], dtype=out.dtype, device=device)
    for r0 in range(0, out.shape[0], stage.shape[0]):
        r1 = min(out.shape[0], r0 + stage.shape[0])
        fill_features(stage[: r1 - r0], cfg.d, cfg.dist, seed, row0=r0)
        out[r0:r1].copy_(stage[: r1 - r0])
    torch.cuda.synchronize(device)


def presample_seeds(cfg: WorkloadConfig, batches: int, device="cpu") -> torch.Tensor:
    """Seeds for pre-sampling the feature cache's hotness: the last `batches` whole batches of epoch
    0's seed order, which a measurement that starts at the front of the epoch does not reach."""
    order = epoch_seed_order(cfg, 0, device)
    n = batches * cfg.batch
    if n > order.numel():
        raise ValueError("more pre-sampling seeds than nodes")
    return order[order.numel() - n:]


def epoch_seed_order(cfg: WorkloadConfig, epoch: int = 0, device="cpu") -> torch.Tensor:
    """Seed nodes of one epoch, in batch order (int32).  With n_train, the training set is the first
    n_train nodes of a seeded node order, reshuffled per epoch; otherwise the whole seeded order."""
    order = node_order(cfg.num_nodes, sub_seed(cfg.rng_seed, 3), device)
    if cfg.n_train is None:
        return order.to(torch.int32)
    train = order[: cfg.n_train]
    k = torch.arange(cfg.n_train, dtype=torch.int64, device=device)
    es = sub_seed(cfg.rng_seed, 5) ^ (epoch * 0x9E3779B97F4A7C15 & 0xFFFFFFFFFFFFFFFF)
    perm = torch.argsort(u32(es, k) * (1 << 31) + k)
    return train[perm].to(torch.int32)


def batch_seeds(order: torch.Tensor, batch: int, b: int) -> torch.Tensor:
    """Seeds of batch b (the last batch of an epoch may be short)."""
    return order[b * batch: (b + 1) * batch]
