"""Test-side helpers: hand-built graphs, a textbook BFS, golden-file parsing.  No method arithmetic
of either side lives here."""
from __future__ import annotations

import os
from fractions import Fraction
from typing import Dict, List

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def csr_from_rows(rows: List[List[int]], indptr_dtype=np.int32):
    """CSR by destination from explicit row lists (row v = sources of edges into v)."""
    indptr = np.zeros(len(rows) + 1, dtype=np.int64)
    for v, r in enumerate(rows):
        indptr[v + 1] = indptr[v] + len(r)
    indices = np.array([u for r in rows for u in r], dtype=np.int32)
    return indptr.astype(indptr_dtype), indices


def star(D: int):
    """Node 0 has in-neighbours 1..D; the leaves have node 0 as their one in-neighbour."""
    return csr_from_rows([list(range(1, D + 1))] + [[0] for _ in range(D)])


def path(n: int):
    """Node v has in-neighbours v-1 and v+1 (where they exist)."""
    return csr_from_rows([[u for u in (v - 1, v + 1) if 0 <= u < n] for v in range(n)])


def complete(n: int):
    return csr_from_rows([[u for u in range(n) if u != v] for v in range(n)])


def random_csr(n: int, avg_deg: float, seed: int, max_deg: int = 64, indptr_dtype=np.int32):
    """Small random CSR with sorted rows, possibly repeated entries and self-loops."""
    rng = np.random.default_rng(seed)
    deg = np.minimum(rng.geometric(1.0 / (avg_deg + 1), size=n) - 1, max_deg)
    rows = [sorted(rng.integers(0, n, size=int(d)).tolist()) for d in deg]
    return csr_from_rows(rows, indptr_dtype)


def bfs_layers(indptr, indices, seeds, hops: int) -> List[np.ndarray]:
    """Textbook BFS along in-edges: layer l = nodes within l steps of the seeds, ascending."""
    seen = set(int(s) for s in seeds)
    frontier = list(seen)
    out = []
    for _ in range(hops):
        nxt = []
        for v in frontier:
            for u in indices[indptr[v]:indptr[v + 1]]:
                u = int(u)
                if u not in seen:
                    seen.add(u)
                    nxt.append(u)
        frontier = nxt
        out.append(np.array(sorted(seen), dtype=np.int32))
    return out


def mean_operator(indptr, indices, n: int) -> np.ndarray:
    """Dense P = D^-1 A with P[v, u] = (multiplicity of u in row v) / deg(v); zero rows stay 0."""
    P = np.zeros((n, n), dtype=np.float64)
    for v in range(n):
        r = indices[indptr[v]:indptr[v + 1]]
        for u in r:
            P[v, u] += 1.0 / len(r)
    return P


def read_golden_splitmix():
    seed, vals = None, []
    with open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("seed"):
                seed = int(line.split()[1])
            else:
                vals.append(int(line))
    return seed, vals


def read_hand_graph():
    rows: Dict[int, List[int]] = {}
    xs: Dict[int, List[float]] = {}
    cases: Dict[str, Dict[str, list]] = {}
    n = 0
    with open(os.path.join(GOLDEN, "hand_graph.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("nodes"):
                n = int(line.split()[1])
            elif line.startswith("row"):
                head, _, rest = line.partition(":")
                rows[int(head.split()[1])] = [int(t) for t in rest.split()]
            elif line.startswith("x "):
                head, _, rest = line.partition(":")
                xs[int(head.split()[1])] = [float(t) for t in rest.split()]
            elif line.startswith("case"):
                parts = line.split()
                name, key = parts[1], parts[2]
                c = cases.setdefault(name, {})
                if key == "seeds":
                    i = parts.index("fanouts")
                    c["seeds"] = [int(t) for t in parts[3:i]]
                    c["fanouts"] = [int(t) for t in parts[i + 1:]]
                elif key.startswith("h"):
                    c[key] = [Fraction(t) for t in parts[3:]]
                else:
                    c[key] = [int(t) for t in parts[3:]]
    indptr, indices = csr_from_rows([rows[v] for v in range(n)])
    x = np.array([xs[v] for v in range(n)], dtype=np.float32)
    return indptr, indices, x, cases
