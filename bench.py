"""Benchmark of the GNN mini-batch hot path on one MI355X.

A step is one pass of the whole path over one mini-batch: k-hop sampling + relabel for every hop,
the feature gather of V_K, and the mean aggregation of every block, all in the library's HIP
kernels.  Inputs (graph, feature table, the epoch's seeds) are resident in HBM before timing.

Prints one JSON line: throughput in sampled edges per second of whole-step time (steps issued round
robin on a few streams, as an epoch would run; the single-stream figure beside it), the stage times,
the gathered-feature bandwidth, the roofline of the dominant kernel (algorithmic bytes / its
HIP-event-timed average duration, against the 8 TB/s HBM3E peak) and the oracle's CPU baseline on
a bounded sample of the same batches.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# Plain-ALU ceiling of the sampler's hashing: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3e12
# lane-instructions/s (one wave64 VALU instruction per SIMD every 4 clocks), over the 19 VALU
# instructions per key of the candidate loop (gfx950 assembly of k_sample: 76 per four keys --
# four SplitMix64 finalisers of 16 instructions each on the key's high word, three 64-bit counter
# adds, four 32-bit compares and five of loop bookkeeping).
ALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
VALU_PER_KEY = 19.0
KEYS_PEAK_MODEL = ALU_LANE_OPS / VALU_PER_KEY
PRESAMPLE_BATCHES = 64     # batches pre-sampled to rank the hot-row cache (disjoint seeds)


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload_name(cfg) -> str:
    return (f"{cfg.name}: R-MAT ({cfg.rmat[0]},{cfg.rmat[1]},{cfg.rmat[2]}) {cfg.num_nodes} nodes, "
            f"{cfg.num_edges} directed edges, int{8 * cfg.indptr_bytes} indptr; {cfg.d}-d fp32 "
            f"{'N(0,1)' if cfg.dist == 'normal' else 'U[-1,1]'} features (row stride {cfg.ld}); "
            f"batch {cfg.batch}; fanouts {cfg.fanouts}" +
            (f"; epoch of {cfg.n_train} training seeds" if cfg.n_train else ""))


def kernel_instance(kind: str, d: int, ld: int, batched: bool, union: bool = False) -> str:
    """Name of the template instance the library launches for this row shape: both kernels pick
    lanes per row (16, 32 or 64) and, with 64, chunk groups per lane (up to 4) from the 16-byte
    chunks per row, and keep a ring of rows (gather: 8 with 64 lanes, else 4) or edges (mean: 4
    with one chunk group per lane, 2 with more) in flight; a gather of rows that are not 16-byte aligned takes the flat per-element kernel.
    Batched, one gather launch serves every sub-batch (k_gather_batch); through the union of the
    sub-batches' node sets, the row engine scatters each union row to its sub-batches."""
    cpr = (d + 3) // 4
    G = 16 if cpr <= 16 else (32 if cpr <= 32 else 64)
    CH = 1 if G < 64 else min(4, (cpr + 63) // 64)
    if kind == "gather":
        if ld % 4:
            return "k_gather<1, 4>"
        R = 8 if G == 64 else 4
        if union:
            return f"k_gather_rows<{G}, {CH}, {R}, true>"
        return f"{'k_gather_batch' if batched else 'k_gather_rows'}<{G}, {CH}, {R}>"
    return f"k_mean_v5<{G}, {CH}, {4 if CH == 1 else 2}>"


def batched_gather(cfg, layout: str) -> bool:
    """The library's gather layout: batched unless interleaving is asked for."""
    return layout != "interleaved"


UNION_GATHER_MIN_D = 128   # rows wider than this, from a table in HBM: the union gather


def union_gather(cfg, layout: str, G: int) -> bool:
    """Whether the library gathers a super-batch through the union of its node sets."""
    return (batched_gather(cfg, layout) and not cfg.host_features and not cfg.cache_bytes
            and G > 1 and cfg.d > UNION_GATHER_MIN_D and cfg.ld % 4 == 0)


def algorithmic_bytes(counts, n_seeds, d, K):
    """Per-launch algorithmic HBM bytes of the gather (a4) and of each mean block (a5).

    a4: |V_K| * (4 + 2*d*4)          read the id, read the row, write the row
    a5 block l: |V_l|*d*4 (each source row once) + |E_l|*4 + (|V_{l-1}|+1)*4 + |V_{l-1}|*d*4
    """
    E = [counts[2 * l] for l in range(K)]
    V = [counts[2 * l + 1] for l in range(K)]
    Vm = [n_seeds] + V          # Vm[l] = |V_l|, l = 0..K
    gather = V[K - 1] * (4 + 2 * d * 4)
    mean = [Vm[l] * d * 4 + E[l - 1] * 4 + (Vm[l - 1] + 1) * 4 + Vm[l - 1] * d * 4
            for l in range(1, K + 1)]
    return gather, mean, E, V


# Mini-batches per super-batch where the workload does not fix it: the largest the library takes
# (sharing grows with it; dense 1849 -> 2117M, 111M-node 1351 -> 1653M, billion-edge 1732 ->
# 1940M sampled edges/s from 8 to 16).
DEFAULT_GROUP = 16


def super_batch_size(cfg, requested: int) -> int:
    """The super-batch size of a run: the one asked for, else the workload's own, else
    DEFAULT_GROUP."""
    if requested:
        return requested
    return cfg.group if cfg.group > 1 else DEFAULT_GROUP


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default: five epochs, or 100 super-batches)")
    ap.add_argument("--group", type=int, default=0,
                    help="mini-batches per super-batch (one step = one super-batch); default: the "
                         "workload's own where its definition fixes one (mid: 8), else "
                         f"{DEFAULT_GROUP}")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="large",
                    help="workload (synth.CONFIGS); default: the largest that fits one GPU's HBM, "
                         "111M nodes / 1.6B edges / 128-d")
    ap.add_argument("--streams", type=int, default=1,
                    help="streams of the single-stream regions (the stage and kernel timings)")
    ap.add_argument("--pipeline-streams", type=int, default=3,
                    help="HIP streams the headline issues the super-batches on, round robin; each "
                         "has its own workspace and outputs, so one stream's sampling overlaps "
                         "another's gather and aggregation (3 measured best of 2, 3, 4 and 6; "
                         "0 or 1: the headline is the single-stream region)")
    ap.add_argument("--superbatch", default="auto", choices=["auto", "full", "compact"],
                    help="super-batch relabel mode (identical results)")
    ap.add_argument("--gather", default="auto", choices=["auto", "interleaved", "batched"],
                    help="gather / outermost-mean launch layout (identical results)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-g1", action="store_true",
                    help="skip the region that times the same mini-batches one per call (G = 1)")
    ap.add_argument("--fanouts", default="",
                    help="comma-separated fanouts replacing the workload's (fanouts[0] at hop 1), "
                         "e.g. 5,10,15 for GARDEN's fanout-pattern sweep")
    ap.add_argument("--no-sage", action="store_true",
                    help="skip the GraphSAGE-mean layer measurement")
    ap.add_argument("--host-indices", action="store_true",
                    help="the graph's neighbour ids in pinned host memory, read in place by the "
                         "sampler (indptr stays in HBM)")
    ap.add_argument("--dyn-passes", type=int, default=-1,
                    help="Dynamic-Cache region: passes of --steps fresh super-batches each, measured "
                         "with the static cache alone and then with the Dynamic-Cache on (default: 4 "
                         "for a workload with host-resident features, else 0 = off)")
    ap.add_argument("--cache-gb", type=float, default=-1.0,
                    help="static hot-row cache size in GB replacing the workload's (a sensitivity "
                         "run; the workload's own size is the measured configuration)")
    ap.add_argument("--dyn-gamma", type=float, default=DYN_GAMMA)
    ap.add_argument("--dyn-rows", type=int, default=0,
                    help="Dynamic-Cache rows (default: 1/8 of the static cache's rows)")
    ap.add_argument("--dyn-t-update", type=int, default=0,
                    help="mini-batches between refreshes (default: one super-batch)")
    ap.add_argument("--dyn-max-refreshes", type=int, default=0)
    ap.add_argument("--match-window", type=int, default=8,
                    help="Match + Greedy Reorder region: a window of this many consecutive "
                         "mini-batches (G = 1), gathered plainly, with Match in sampling order and "
                         "with Match in greedy order (0 = off; at most 16)")
    ap.add_argument("--adj-cache-gb", type=float, default=0.0,
                    help="with --host-indices: an HBM adjacency cache of this many GB of "
                         "pre-sampled hot rows")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU: the mini-batch path is measured on "
                                   "one MI355X; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import graph_mini_pipeline_amd as gm
    import synth

    cfg = synth.CONFIGS[args.config]
    if args.fanouts:
        import dataclasses
        cfg = dataclasses.replace(cfg, fanouts=[int(f) for f in args.fanouts.split(",")])
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    graph = synth.build_graph(cfg, device=dev)
    torch.cuda.synchronize()
    progress(f"graph: {cfg.num_nodes} nodes, {graph.indices.numel()} edges in {time.perf_counter() - t0:.1f} s")
    if cfg.host_features:
        table = torch.empty(cfg.num_nodes, cfg.ld, dtype=torch.float32, pin_memory=True)
        synth.make_features(cfg, table, device=dev)
    else:
        table = torch.empty(cfg.num_nodes, cfg.ld, dtype=torch.float32, device=dev)
        synth.make_features(cfg, table)
    order = synth.epoch_seed_order(cfg, 0, device=dev).contiguous()
    n_batches = (order.numel() + cfg.batch - 1) // cfg.batch
    G = super_batch_size(cfg, args.group)
    n_super = (n_batches + G - 1) // G
    # default: five epochs for a workload with a training set (each epoch its own seed order),
    # else 100 super-batches (30 with a host-resident table), wrapping round a short seed order
    # with a fresh batch seed per step
    steps = args.steps or (5 * n_super if cfg.n_train else (30 if cfg.host_features else 100))
    # seed order of each epoch the steps reach, made before any timing
    orders = [order] + [synth.epoch_seed_order(cfg, e, device=dev).contiguous()
                        for e in range(1, (steps + n_super - 1) // n_super)]
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t0
    progress(f"features ({'pinned host' if cfg.host_features else 'HBM'}) and {len(orders)} seed "
             f"order(s) ready, {t_gen:.1f} s in all")
    K = len(cfg.fanouts)

    dg = gm.DeviceGraph(cfg.num_nodes, graph.indptr, graph.indices)
    adj = None          # host-resident neighbour ids: what the adjacency cache holds
    if args.host_indices:
        from graph_mini_pipeline_amd.hotness import presample_adjacency_order
        t1 = time.perf_counter()
        ind_host = torch.empty(graph.indices.numel(), dtype=torch.int32, pin_memory=True)
        ind_host.copy_(graph.indices)
        adj_entries = int(args.adj_cache_gb * 1e9) // 4
        adj_cache, cached = None, torch.zeros(cfg.num_nodes, dtype=torch.bool, device=dev)
        if adj_entries:
            pre = synth.presample_seeds(cfg, PRESAMPLE_BATCHES, device=dev)
            if pre.numel() // cfg.batch + steps * G > n_batches:
                raise SystemExit("pre-sampling seeds would overlap the measured batches")
            adj_hot = presample_adjacency_order(dg, graph.indptr, pre, cfg.batch, cfg.fanouts,
                                                synth.sub_seed(cfg.rng_seed, 7))
            adj_cache = gm.gnn_adjacency_cache_create(
                gm.DeviceGraph(cfg.num_nodes, graph.indptr, ind_host), adj_hot, adj_entries)
            # the cache holds the longest prefix of the order that fits (the library's rule)
            dh = (graph.indptr[1:] - graph.indptr[:-1])[adj_hot.long()]
            m = int((torch.cumsum(dh, 0) <= adj_entries).sum().item())
            cached[adj_hot[:m].long()] = True
        graph = synth.Graph(graph.num_nodes, graph.indptr, ind_host)   # ids leave HBM
        torch.cuda.empty_cache()
        dg = gm.DeviceGraph(cfg.num_nodes, graph.indptr, ind_host, adjacency=adj_cache)
        adj = {"cached": cached, "cache": adj_cache, "entries": adj_entries,
               "setup_s": time.perf_counter() - t1, "rows_read": 0, "rows_hit": 0,
               "ids_read": 0, "ids_hit": 0}
        progress(f"neighbour ids in pinned host memory; adjacency cache "
                 f"{adj_cache.rows if adj_cache else 0} rows, "
                 f"{adj_cache.entries if adj_cache else 0} ids, {adj['setup_s']:.1f} s")
    cache_rows, t_rank = 0, 0.0
    hot_order = None
    if args.cache_gb >= 0:
        import dataclasses
        cfg = dataclasses.replace(cfg, cache_bytes=int(args.cache_gb * 1e9))
    if cfg.cache_bytes:
        from graph_mini_pipeline_amd.hotness import presample_hot_order
        t1 = time.perf_counter()
        cache_rows = min(cfg.num_nodes, cfg.cache_bytes // (cfg.ld * 4))
        pre = synth.presample_seeds(cfg, PRESAMPLE_BATCHES, device=dev)
        if pre.numel() // cfg.batch + steps * G > n_batches:
            raise SystemExit("pre-sampling seeds would overlap the measured batches")
        hot_order = presample_hot_order(dg, graph.indptr, pre, cfg.batch, cfg.fanouts,
                                        synth.sub_seed(cfg.rng_seed, 6), cache_rows)
        t_rank = time.perf_counter() - t1
        progress(f"hot-row order: {PRESAMPLE_BATCHES} pre-sampled batches, {cache_rows} cache rows, "
                 f"{t_rank:.1f} s")
    fs = gm.gnn_feature_store_create(table, cfg.d, cache_rows, hot_order)
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, cfg.num_nodes)
    S = max(1, args.streams)
    P = max(0, args.pipeline_streams)
    P = P if P > 1 else 0
    # streams 0..S-1 (0: the default stream) time the single-stream regions and the kernels; the
    # pipelined headline has streams S..S+P-1 of its own, so a kernel trace separates the two
    wss = [torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes, G), dtype=torch.uint8, device=dev)
           for _ in range(S + P)]
    streams = [None] + [torch.cuda.Stream(device=dev) for _ in range(S + P - 1)]
    outs = [{} for _ in range(S + P)]   # per stream: one output set per (position, seed count)

    def batch_range(s):
        b0 = s * G
        return list(range(b0, min(b0 + G, n_batches)))

    def step(st, timer=None, first=0, ns=S):
        """Step st: super-batch st mod n_super of epoch st div n_super, on stream first + st % ns;
        its batches share the batch seed of step st.  Returns (st, [(b, n, out)], its seeds)."""
        e, s = divmod(st, n_super)
        od = orders[e % len(orders)]
        q = first + st % ns
        bs = batch_range(s)
        lo = bs[0] * cfg.batch
        hi = min(od.numel(), (bs[-1] + 1) * cfg.batch)
        ptr = [min(b * cfg.batch, od.numel()) - lo for b in bs] + [hi - lo]
        mine = []
        for j, b in enumerate(bs):
            n = ptr[j + 1] - ptr[j]
            if (j, n) not in outs[q]:
                outs[q][(j, n)] = gm.MinibatchOut(gm.gnn_capacity(n, cfg.fanouts, cfg.num_nodes),
                                                  cfg.d, cfg.ld, stream=streams[q])
            mine.append((b, n, outs[q][(j, n)]))
        gm.gnn_minibatch(dg, fs, od[lo:hi], ptr, cfg.fanouts, gm.gnn_batch_seed(cfg.rng_seed, st),
                         [m[2] for m in mine], wss[q], gm.Options(superbatch=args.superbatch, gather=args.gather),
                         timer=timer, stream=streams[q])
        return st, mine, od[lo:hi]

    torch.cuda.synchronize()
    for b in range(max(args.warmup, S)):
        step(b)
    torch.cuda.synchronize()
    assert all(gm.gnn_read_device_status(w) == gm.GNN_OK for w in wss[:S])

    # Timed region 1, the headline: the steps issued round robin on P streams, each with its own
    # workspace and outputs, so that one super-batch's sampling (ALU and latency bound) overlaps
    # another's gather and aggregation (HBM bound) -- the throughput of an epoch as a training
    # loop would run it.  Each step is still the whole path over its super-batch.
    wall_p = None
    if P:
        for b in range(P):
            step(b, first=S, ns=P)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for b in range(steps):
            step(b, first=S, ns=P)
        torch.cuda.synchronize()
        wall_p = time.perf_counter() - t0
        progress(f"pipelined region ({P} streams): {steps} steps in {wall_p:.3f} s")

    # Timed region 2: the same steps one after another on one stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for b in range(steps):
        step(b)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    status = min(gm.gnn_read_device_status(w) for w in wss)
    progress(f"single-stream region: {steps} steps in {wall:.3f} s")

    # Timed region 3: region 2 with HIP events at the stage boundaries, for the per-kernel times
    # (the events cost a few microseconds each, so they stay out of regions 1 and 2).
    timer = gm.Timer(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for b in range(steps):
        step(b, timer)
    torch.cuda.synchronize()
    wall_events = time.perf_counter() - t0
    stages = np.array(timer.elapsed(), dtype=np.float64)      # [steps, 5] ms
    head_wall = wall_p if wall_p is not None else wall
    head_streams = P if wall_p is not None else S

    # Region 4: the same mini-batches, one per call (G = 1), issued round robin on the headline's
    # streams with workspaces and outputs of their own: what the super-batch adds over plain
    # mini-batches.  Each mini-batch takes the batch seed of its global index.
    g1 = None
    if G > 1 and not args.no_g1:
        mbs = []
        for st in range(steps):
            e, sb = divmod(st, n_super)
            od = orders[e % len(orders)]
            for b in batch_range(sb):
                lo, hi = b * cfg.batch, min(od.numel(), (b + 1) * cfg.batch)
                mbs.append((od[lo:hi], gm.gnn_batch_seed(cfg.rng_seed, st * G + b - sb * G)))
        Q = max(1, P)
        qs = streams[S:S + P] if P else [streams[0]]
        ws1 = [torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes, 1), dtype=torch.uint8,
                           device=dev) for _ in range(Q)]
        outs1 = [{} for _ in range(Q)]

        def step1(i):
            sd, seed = mbs[i]
            q = i % Q
            n = sd.numel()
            if n not in outs1[q]:
                outs1[q][n] = gm.MinibatchOut(gm.gnn_capacity(n, cfg.fanouts, cfg.num_nodes),
                                              cfg.d, cfg.ld, stream=qs[q])
            gm.gnn_minibatch(dg, fs, sd, [0, n], cfg.fanouts, seed, [outs1[q][n]], ws1[q],
                             gm.Options(gather=args.gather), stream=qs[q])
            return outs1[q][n]

        for i in range(min(len(mbs), 2 * Q)):
            step1(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(len(mbs)):
            step1(i)
        torch.cuda.synchronize()
        wall1 = time.perf_counter() - t0
        assert all(gm.gnn_read_device_status(w) == gm.GNN_OK for w in ws1)
        edges1 = 0
        for i in range(len(mbs)):     # untimed: the sampled edges of each mini-batch
            o = step1(i)
            torch.cuda.synchronize()
            cnt = o.blocks.counts.cpu().tolist()
            edges1 += sum(cnt[2 * l] for l in range(K))
        g1 = {"value": edges1 / wall1, "unit": "sampled edges/s", "streams": Q,
              "minibatches": len(mbs), "ms_per_minibatch": wall1 / len(mbs) * 1e3,
              "note": "the same mini-batches, one per gnn_minibatch call (no super-batch), each "
                      "with the batch seed of its global index, round robin on the headline's "
                      "streams"}
        progress(f"G = 1 region: {len(mbs)} mini-batches in {wall1:.3f} s")

    # Sizes of each timed batch: sampling is a pure function of the batch, so an untimed re-run
    # of the sampling gives the counts.
    tot_edges = 0
    gb_bytes = []      # bytes the gather launch moves (the union gather: its own, fewer)
    gb_defined = []    # the gather's algorithmic bytes by the per-mini-batch definition
    mean_bytes = []
    payload = []
    hits = torch.zeros(1, dtype=torch.int64, device=dev)
    rows_gathered = 0
    keys = 0      # sampling keys hashed: over each hop's union frontier, the degrees above the fanout
    deg = (graph.indptr[1:] - graph.indptr[:-1]).to(torch.int32)
    union = union_gather(cfg, args.gather, G)
    for b in range(steps):
        _, mine, sb_seeds = step(b)
        torch.cuda.synchronize()
        if union:   # the union gather reads each row of U_K once and writes every sub-batch row
            vk = [out.blocks.nodes[K - 1][:int(out.blocks.counts[2 * K - 1].item())] for _, _, out in mine]
            n_union = int(torch.unique(torch.cat(vk)).numel())
            rows = sum(int(v.numel()) for v in vk)
            gb_union = n_union * (4 + cfg.d * 4 + G * 4) + rows * cfg.d * 4
        for l in range(K):
            if l == 0:   # the seeds of the super-batch
                fr = [sb_seeds]
            else:        # each sub-batch's V_{l-1}
                fr = [out.blocks.nodes[l - 1][:int(out.blocks.counts[2 * l - 1].item())]
                      for _, _, out in mine]
            u = torch.unique(torch.cat(fr).long())
            dd = deg[u]
            keys += int(dd[dd > cfg.fanouts[l]].sum().item())
            if adj is not None:   # rows the sampler reads: ids min(deg, k) of each, cached or not
                ids = dd.clamp(max=cfg.fanouts[l])
                hit = adj["cached"][u]
                adj["rows_read"] += int((dd > 0).sum().item())
                adj["rows_hit"] += int(((dd > 0) & hit).sum().item())
                adj["ids_read"] += int(ids.sum().item())
                adj["ids_hit"] += int(ids[hit].sum().item())
        g_s, m_s, p_s = 0, [0] * K, 0
        for _, n, out in mine:
            if cache_rows:   # hits of this batch's gather: the same gather again, counting
                gm.gnn_gather_features(fs, out.blocks.nodes[K - 1], out.x,
                                       d_n=out.blocks.counts[2 * K - 1:2 * K], d_hits=hits)
            cnt = out.blocks.counts.cpu().tolist()
            rows_gathered += cnt[2 * K - 1]
            g_b, m_b, E, V = algorithmic_bytes(cnt, n, cfg.d, K)
            tot_edges += sum(E)
            g_s += g_b
            m_s = [x + y for x, y in zip(m_s, m_b)]
            p_s += V[K - 1] * cfg.d * 4
        gb_bytes.append(gb_union if union else g_s)
        gb_defined.append(g_s)
        mean_bytes.append(m_s)
        payload.append(p_s)
    gb_bytes = np.array(gb_bytes, dtype=np.float64)
    gb_defined = np.array(gb_defined, dtype=np.float64)
    mean_outer = np.array([m[K - 1] for m in mean_bytes], dtype=np.float64)
    mean_all = np.array([sum(m) for m in mean_bytes], dtype=np.float64)

    keys_peak = hash_ceiling(gm, dev)
    progress(f"hash ceiling: {keys_peak / 1e12:.2f}e12 keys/s")
    n_minibatches = sum(len(batch_range(b % n_super)) for b in range(steps))
    batched = batched_gather(cfg, args.gather)
    launches = 1 if batched else G      # gather (and outermost-mean) launches per step
    # shared outermost means: batched from a table in HBM without a cache, G > 1: one mean launch
    # over the union frontier, storing each node's mean to every sub-batch that holds it
    shared = batched and not cfg.host_features and not cfg.cache_bytes and G > 1
    t_sample, t_gather, t_mean_outer, t_mean_rest, t_hash = (stages[:, i].sum() / 1e3 for i in range(5))
    kern = {
        "gather": (gb_bytes.sum() / t_gather / 1e9, t_gather / steps / launches * 1e3),
        "mean_outer": (mean_outer.sum() / t_mean_outer / 1e9, t_mean_outer / steps / launches * 1e3),
    }
    dom = "gather" if t_gather >= t_mean_outer else "mean_outer"
    ach, avg_ms = kern[dom]
    # per mini-batch: every batch's a4 + a5 bytes over the stage times (with the union gather the
    # bytes it moves itself, fewer, are reported beside it)
    t_ga = t_gather + t_mean_outer + t_mean_rest
    ga_frac = (gb_defined.sum() + mean_all.sum()) / t_ga / 1e9 / HBM_PEAK_GBPS
    ga_frac_moved = (gb_bytes.sum() + mean_all.sum()) / t_ga / 1e9 / HBM_PEAK_GBPS
    names = {"gather": kernel_instance("gather", cfg.d, cfg.ld, batched, union),
             "mean_outer": kernel_instance("mean", cfg.d, cfg.ld, batched)}
    stage_kernels = {"gather": (f"{names['gather']}: each row of the union of the sub-batches' "
                                f"V_K read once, stored to every sub-batch that holds it"
                                if union else names["gather"]),
                     "mean_outer": (f"{names['mean_outer']} over the union frontier, each row "
                                    f"stored to every sub-batch that holds it"
                                    if shared else names["mean_outer"])}
    other = "mean_outer" if dom == "gather" else "gather"
    from graph_mini_pipeline_amd.rocprof_summary import read_traffic
    counters = os.path.join(ROOT, "profiles", f"{cfg.name}_counters.txt")
    traffic = {"gather": read_traffic(counters, names["gather"]),
               "mean_outer": read_traffic(counters, names["mean_outer"] + "@outer")}
    alg_per_launch = {"gather": gb_bytes.sum() / steps / launches,
                      "mean_outer": mean_outer.sum() / steps / launches}

    result = {
        "metric": "sampled edges/s + gathered feature GB/s per mini-batch; % of HBM peak",
        "value": tot_edges / head_wall,
        "unit": "sampled edges/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": head_wall / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload_name(cfg), "batches_per_epoch": n_batches,
                   "super_batch": G, "streams": head_streams, "superbatch_relabel": args.superbatch,
                   "gather_layout": args.gather,
                   "step": f"one super-batch of {G} mini-batch(es)"},
        "ms_per_minibatch": head_wall / n_minibatches * 1e3,
        "status": gm.gnn_status_string(status),
        "sampled_edges_per_s_sampling_stage": tot_edges / t_sample,
        "gathered_GBps": float(np.sum(payload) / t_gather / 1e9),
        "gather_aggregate_hbm_frac": ga_frac,
        "gather_aggregate_hbm_frac_moved_bytes": ga_frac_moved,
        "stage_ms_per_step": {"sample_relabel": t_sample / steps * 1e3,
                              "gather": t_gather / steps * 1e3,
                              "mean_outer_block": t_mean_outer / steps * 1e3,
                              "mean_other_blocks": t_mean_rest / steps * 1e3,
                              "sampling_kernel_only": t_hash / steps * 1e3},
        "roofline": {"bound": "hbm", "kernel": stage_kernels[dom],
                     "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBPS,
                     "traffic": traffic[dom]["bytes"] if traffic[dom] else None,
                     "algorithmic_bytes_per_launch": alg_per_launch[dom],
                     "avg_launch_ms": avg_ms, "launches_per_step": launches},
        "sampler": {"bound": "alu", "kernel": "k_sample", "achieved": keys / t_hash,
                    "peak": keys_peak, "unit": "keys/s", "frac": keys / t_hash / keys_peak,
                    "keys_per_step": keys / steps, "ms_per_step": t_hash / steps * 1e3,
                    "peak_source": "measured in this run: gnn_hash_probe (the key hashing alone, "
                                   "every lane of a full grid), best of 3 launches",
                    "peak_model": KEYS_PEAK_MODEL,
                    "frac_of_model": keys / t_hash / KEYS_PEAK_MODEL,
                    "peak_model_derivation": "256 CU x 4 SIMD x 16 lanes x 2.4 GHz / 19 VALU "
                                             "instructions per key of the candidate loop"},
        "other_kernel": {"name": stage_kernels[other], "achieved_GBps": kern[other][0],
                         "avg_launch_ms": kern[other][1], "launches_per_step": launches,
                         "algorithmic_bytes_per_launch": alg_per_launch[other],
                         "traffic": traffic[other]["bytes"] if traffic[other] else None},
        "ms_per_step_with_stage_events": wall_events / steps * 1e3,
        "stage_ms_percentiles": percentiles(stages),
        "single_stream": {"streams": S, "value": tot_edges / wall, "unit": "sampled edges/s",
                          "ms_per_step": wall / steps * 1e3,
                          "ms_per_minibatch": wall / n_minibatches * 1e3,
                          "note": "the same steps one after another on one stream; the stage and "
                                  "kernel timings come from this layout (with events)"},
        "input_generation_s": t_gen,
        "system": system_fingerprint(dev),
    }

    # Counter calibration: one plain 1 GiB device copy by k_copy_probe (untimed).  Profiling runs
    # of this command read its fetched / written bytes to scale the other kernels' counters.
    probe_src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    probe_dst = torch.empty_like(probe_src)
    gm.gnn_copy_probe(probe_src, probe_dst)
    torch.cuda.synchronize()
    result["copy_probe_bytes"] = probe_src.numel() * 4
    if g1 is not None:
        result["g1"] = g1
    if adj is not None:
        c = adj["cache"]
        result["config"]["neighbour_ids"] = "pinned host memory, read in place"
        result["adjacency"] = {
            "cache_rows": c.rows if c else 0, "cache_ids": c.entries if c else 0,
            "cache_GB": (c.entries if c else 0) * 4 / 1e9,
            "cache_fraction_of_edges": (c.entries if c else 0) / max(1, graph.indices.numel()),
            "ranking": f"{PRESAMPLE_BATCHES} pre-sampled batches from seeds the measurement does "
                       f"not use; host reads saved per cached id, sum over hops of (batches whose "
                       f"frontier holds the node) * min(deg, k) / deg, desc; then the rows not "
                       f"reached, by out-degree * min(deg, max k) / deg, desc" if c else None,
            "setup_s": adj["setup_s"],
            "hit_rate_rows": adj["rows_hit"] / max(1, adj["rows_read"]),
            "hit_rate_ids": adj["ids_hit"] / max(1, adj["ids_read"]),
            "host_ids_per_step": (adj["ids_read"] - adj["ids_hit"]) / steps}
    del probe_src, probe_dst

    if cfg.host_features:
        n_hits = int(hits.item())
        miss_bytes = (rows_gathered - n_hits) * cfg.d * 4
        link = host_link(gm, table, dev)
        miss_rate = miss_bytes / t_gather / 1e9
        result["cache"] = {"rows": cache_rows, "bytes": cache_rows * cfg.ld * 4,
                           "fraction_of_rows": cache_rows / cfg.num_nodes,
                           "ranking": f"{PRESAMPLE_BATCHES} pre-sampled batches from seeds the "
                                      f"measurement does not use; (count desc, degree desc, id asc)",
                           "ranking_s": t_rank,
                           "hit_rate": n_hits / max(1, rows_gathered)}
        result["host_link"] = dict(link, miss_GB_per_step=miss_bytes / steps / 1e9,
                                   miss_GBps_during_gather=miss_rate,
                                   frac=miss_rate / link["B_link_GBps"])
        # the gather's misses cross the host link: that link, not HBM, bounds the dominant kernel
        result["roofline_hbm"] = result["roofline"]
        result["roofline"] = {"bound": "host-link", "kernel": names["gather"],
                              "achieved": miss_rate, "peak": link["B_link_GBps"], "unit": "GB/s",
                              "frac": miss_rate / link["B_link_GBps"], "traffic": None,
                              "peak_source": "measured: best of 5 hipMemcpyAsync of 1 GiB pinned host -> device",
                              "avg_launch_ms": kern["gather"][1], "launches_per_step": launches}
    if not args.no_sage:
        result["sage_layer"] = sage_layer(gm, cfg, dg, fs, order, dev)
        progress("GraphSAGE layer timed")
    if args.match_window > 1:
        result["match_reorder"] = match_reorder_region(gm, cfg, dg, fs, order, dev,
                                                       min(args.match_window, 16))
        progress("Match + Greedy Reorder region done")
    dyn_passes = args.dyn_passes if args.dyn_passes >= 0 else (4 if cfg.host_features else 0)
    if dyn_passes > 0:
        result["dynamic_cache"] = dynamic_cache_region(gm, cfg, args, dg, fs, order, G, steps,
                                                       cache_rows, hot_order, dyn_passes, dev)
        progress("Dynamic-Cache region done")
    progress("stage timing and counts done")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, graph, table, step, args.cpu_seconds,
                                              tot_edges / head_wall)
    print(json.dumps(result), flush=True)


STAGE_NAMES = ("sample_relabel", "gather", "mean_outer_block", "mean_other_blocks",
               "sampling_kernel_only")


# Dynamic-Cache policy (the pages leave gamma, K_dyn and T_update open); measured on the
# billion-edge workload over gamma 0.98-0.999, T_update 16-128 mini-batches and K_dyn 1/32 to 1/2
# of the static cache's rows: the refresh costs about 0.5 ms whatever its interval, so the longest
# interval measured costs least per step, and the longer memory keeps more of the recurring rows.
DYN_GAMMA = 0.995                # per mini-batch: a node's weight halves after 138 mini-batches
DYN_T_UPDATE_SUPERBATCHES = 8    # refresh interval in super-batches


def dynamic_cache_region(gm, cfg, args, dg, fs, order, G, steps, cache_rows, hot_order, passes,
                         dev):
    """GARDEN Sec. IV.B, eq. (5)-(6), measured: pass r runs super-batches r*steps .. (r+1)*steps-1
    of the seed order (batch seed = super-batch index), one stream.  First every pass with the
    static cache alone: an untimed pass for the sizes, the cache hits and the set of rows it
    misses, then a timed pass.  Then the Dynamic-Cache is enabled on the same store and every
    pass is timed again, the refresh due after each super-batch included, so pass r > 0 runs on a
    cache adapted to passes 0..r-1 (the static cache is never changed).  Misses cross the host
    link; the gathered rows are the same either way."""
    import numpy as np
    import torch
    K = len(cfg.fanouts)
    n_batches = (order.numel() + cfg.batch - 1) // cfg.batch
    if passes * steps * G + PRESAMPLE_BATCHES > n_batches:
        raise SystemExit("Dynamic-Cache passes would reach the pre-sampling seeds")
    k_dyn = args.dyn_rows or max(1, cache_rows // 8)
    t_update = args.dyn_t_update or DYN_T_UPDATE_SUPERBATCHES * G
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, cfg.num_nodes)
    ws = torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes, G), dtype=torch.uint8, device=dev)
    outs = {}
    hits = torch.zeros(1, dtype=torch.int64, device=dev)
    opts = gm.Options(d_hits=hits)
    is_static = torch.zeros(cfg.num_nodes, dtype=torch.bool, device=dev)
    if cache_rows:
        is_static[hot_order[:cache_rows].long()] = True

    def run(sb):
        bs = list(range(sb * G, min(sb * G + G, n_batches)))
        lo, hi = bs[0] * cfg.batch, min(order.numel(), (bs[-1] + 1) * cfg.batch)
        ptr = [b * cfg.batch - lo for b in bs] + [hi - lo]
        mine = []
        for j in range(len(bs)):
            n = ptr[j + 1] - ptr[j]
            if (j, n) not in outs:
                outs[(j, n)] = gm.MinibatchOut(gm.gnn_capacity(n, cfg.fanouts, cfg.num_nodes),
                                               cfg.d, cfg.ld)
            mine.append(outs[(j, n)])
        gm.gnn_minibatch(dg, fs, order[lo:hi], ptr, cfg.fanouts,
                         gm.gnn_batch_seed(cfg.rng_seed, sb), mine, ws, opts)
        return mine

    def timed_pass(r, dynamic):
        ev = []
        hits.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for sb in range(r * steps, (r + 1) * steps):
            run(sb)
            if dynamic:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                gm.gnn_dyn_cache_update(fs)
                e1.record()
                ev.append((e0, e1))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        assert gm.gnn_read_device_status(ws) == gm.GNN_OK
        refresh_ms = sum(a.elapsed_time(b) for a, b in ev)
        return wall, int(hits.item()), refresh_ms

    rows, static_hits, recur, static_wall = [], [], [], []
    prev_miss = None
    for r in range(passes):
        n_rows = 0
        hits.zero_()
        miss = torch.zeros(cfg.num_nodes, dtype=torch.bool, device=dev)
        for sb in range(r * steps, (r + 1) * steps):
            for out in run(sb):
                torch.cuda.synchronize()
                nk = int(out.blocks.counts[2 * K - 1].item())
                vk = out.blocks.nodes[K - 1][:nk].long()
                n_rows += nk
                miss[vk[~is_static[vk]]] = True
        rows.append(n_rows)
        static_hits.append(int(hits.item()))
        if prev_miss is not None:
            recur.append(int((miss & prev_miss).sum().item()) / max(1, int(miss.sum().item())))
        prev_miss = miss
        static_wall.append(timed_pass(r, False)[0])
    del miss, prev_miss
    t1 = time.perf_counter()
    gm.gnn_feature_store_enable_dynamic(fs, args.dyn_gamma, k_dyn, t_update,
                                        max_refreshes=args.dyn_max_refreshes)
    setup_s = time.perf_counter() - t1
    out = []
    for r in range(passes):
        wall, h, refresh_ms = timed_pass(r, True)
        info = gm.gnn_dyn_cache_query(fs)
        miss_s = (rows[r] - static_hits[r]) * cfg.d * 4
        miss_d = (rows[r] - h) * cfg.d * 4
        out.append({
            "pass": r, "superbatches": [r * steps, (r + 1) * steps], "rows": rows[r],
            "static": {"hit_rate": static_hits[r] / max(1, rows[r]),
                       "ms_per_step": static_wall[r] / steps * 1e3,
                       "host_link_GB_per_step": miss_s / steps / 1e9},
            "dynamic": {"hit_rate": h / max(1, rows[r]),
                        "ms_per_step": wall / steps * 1e3,
                        "host_link_GB_per_step": miss_d / steps / 1e9,
                        "refresh_ms_per_step": refresh_ms / steps,
                        "refreshes": info["refreshes"], "members": info["members"],
                        "resident": info["resident"], "last_published": info["last_published"],
                        "last_candidates": info["last_candidates"],
                        "last_admitted": info["last_admitted"],
                        "last_evicted": info["last_evicted"]},
            "static_miss_recurrence": recur[r - 1] if r > 0 else None})
        progress(f"Dynamic-Cache pass {r}: hit rate {static_hits[r] / max(1, rows[r]):.4f} -> "
                 f"{h / max(1, rows[r]):.4f}, {static_wall[r] / steps * 1e3:.2f} -> "
                 f"{wall / steps * 1e3:.2f} ms per step")
    return {"gamma": args.dyn_gamma, "k_dyn": k_dyn, "t_update": t_update,
            "max_refreshes": args.dyn_max_refreshes,
            "rows_GB": k_dyn * cfg.ld * 4 / 1e9,
            "bookkeeping_GB": (cfg.num_nodes * 20 + (cfg.num_nodes + 31) // 32 * 8 + k_dyn * 13) / 1e9,
            "setup_s": setup_s, "passes": out,
            "static_miss_recurrence": "fraction of the distinct nodes missed by the static cache "
                                      "in a pass that it also missed in the pass before",
            "note": "one stream; pass r > 0 runs on the Dynamic-Cache as pass r - 1 left it"}


def match_reorder_region(gm, cfg, dg, fs, order, dev, B):
    """FastGL's Match and Greedy Reorder ("The idea", "What it costs") on B consecutive mini-batches
    of the epoch order, one per call (G = 1): each batch's X gathered plainly, then again with
    Match (rows the previous batch's X holds are copied from it) in sampling order and in the
    greedy nearest-overlap-first order of the batches' overlap matrix.  Reports the share of each
    batch's rows found in its predecessor, the rows read from the store (HBM table or cache; with a
    host table, the misses of the HBM cache cross the host link), the gather times from HIP events,
    and whether every X equals the plain one bit for bit."""
    import numpy as np
    import torch
    K = len(cfg.fanouts)
    N = cfg.num_nodes
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, N)
    ws = torch.empty(gm.gnn_workspace_size(caps, N), dtype=torch.uint8, device=dev)
    blocks = []
    for b in range(B):
        bl = gm.Blocks(caps)
        gm.gnn_sample_khop(dg, order[b * cfg.batch:(b + 1) * cfg.batch], cfg.fanouts,
                           gm.gnn_batch_seed(cfg.rng_seed, b), bl, ws)
        blocks.append(bl)
    torch.cuda.synchronize()
    del ws
    ids = [bl.nodes[K - 1] for bl in blocks]
    cnt = [bl.counts[2 * K - 1:2 * K] for bl in blocks]
    rows = [int(c.item()) for c in cnt]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1)

    ov = torch.empty(B * B, dtype=torch.int64, device=dev)
    t_ov = min(timed(lambda: gm.gnn_batch_overlap(ids, ov, counts=cnt)) for _ in range(3))
    M = ov.cpu().numpy().reshape(B, B)
    t0 = time.perf_counter()
    greedy = gm.gnn_greedy_order(M, 0)
    t_greedy = (time.perf_counter() - t0) * 1e3
    hits = torch.zeros(1, dtype=torch.int64, device=dev)
    X = [torch.empty(max(caps.nodes[K - 1], 1), cfg.ld, dtype=torch.float32, device=dev)
         for _ in range(B)]
    t_plain = sum(timed(lambda i=i: gm.gnn_gather_features(fs, ids[i], X[i], d_n=cnt[i], d_hits=hits))
                  for i in range(B))
    hits_plain = int(hits.item())

    def with_match(o):
        Y = [torch.empty_like(X[0]) for _ in range(B)]
        match = torch.empty(max(caps.nodes[K - 1], 1), dtype=torch.int32, device=dev)
        matched = torch.zeros(1, dtype=torch.int64, device=dev)
        hits.zero_()
        t = 0.0
        for j, i in enumerate(o):
            if j == 0:
                t += timed(lambda: gm.gnn_gather_features(fs, ids[i], Y[i], d_n=cnt[i], d_hits=hits))
            else:
                p = o[j - 1]
                t += timed(lambda: gm.gnn_gather_features_match(
                    fs, ids[i], Y[i], ids[p], Y[p], match, d_n=cnt[i], d_prev_n=cnt[p],
                    d_matched=matched, d_hits=hits))
        same = all(torch.equal(Y[i][:rows[i], :cfg.d], X[i][:rows[i], :cfg.d]) for i in range(B))
        m = int(matched.item())
        follow = sum(rows[i] for i in o[1:])
        r = {"order": list(o), "rows_found_in_predecessor": m,
             "share_of_rows_found": m / max(1, follow),
             "overlap_from_matrix": int(sum(M[o[j - 1], o[j]] for j in range(1, B))),
             "rows_read_from_store": sum(rows) - m,
             "gather_ms_per_batch": t / B, "identical_X": bool(same)}
        if cfg.host_features:
            r["rows_over_host_link"] = sum(rows) - m - int(hits.item())
        del Y
        return r

    seq = with_match(list(range(B)))
    grd = with_match(greedy)
    out = {"window": B, "batches": f"0..{B - 1} of the epoch order, batch seed of each index",
           "rows": sum(rows), "plain_gather_ms_per_batch": t_plain / B,
           "overlap_matrix_ms": t_ov, "greedy_order_host_ms": t_greedy,
           "mean_pairwise_share": float((M.sum() - np.trace(M)) / max(1, (B - 1) * sum(rows))),
           "sampling_order": seq, "greedy_order": grd}
    if cfg.host_features:
        out["plain_rows_over_host_link"] = sum(rows) - hits_plain
    return out


def percentiles(stages):
    """Median, p10 and p90 over the timed steps of each stage and of the whole step (HIP events at
    the stage boundaries, one stream), in ms per step."""
    import numpy as np
    out = {}
    total = stages[:, :4].sum(axis=1)
    for name, col in list(zip(STAGE_NAMES, stages.T)) + [("step", total)]:
        p10, p50, p90 = np.percentile(col, [10, 50, 90])
        out[name] = {"p10": float(p10), "median": float(p50), "p90": float(p90)}
    return out


SAGE_D_OUT = 128            # GraphSAGE hidden width of GARDEN Sec. VI.A
FP32_MFMA_TFLOPS = 157.3    # MI355X dense fp32 matrix peak


def sage_layer(gm, cfg, dg, fs, order, dev, reps=20):
    """One GraphSAGE-mean layer (mean, concat, dense UPDATE to 128 features on fp32 matrix cores)
    over the outermost block of one batch of this workload, X as its source rows.  HIP events on
    the stream the library runs on time the whole layer (gnn_sage_layer), the mean alone and the
    UPDATE alone (gnn_sage_update on the layer's means)."""
    import numpy as np
    import torch
    K = len(cfg.fanouts)
    caps = gm.gnn_capacity(cfg.batch, cfg.fanouts, cfg.num_nodes)
    mo = gm.MinibatchOut(caps, cfg.d, cfg.ld)
    ws = torch.empty(gm.gnn_workspace_size(caps, cfg.num_nodes, 1), dtype=torch.uint8, device=dev)
    gm.gnn_minibatch(dg, fs, order[:cfg.batch].contiguous(), [0, cfg.batch], cfg.fanouts,
                     gm.gnn_batch_seed(cfg.rng_seed, 0), [mo], ws)
    cnt = mo.blocks.counts.cpu().tolist()
    n_dst = cfg.batch if K == 1 else int(cnt[2 * (K - 2) + 1])
    n_edges = int(cnt[2 * (K - 1)])
    indptr = mo.blocks.indptr[K - 1][:n_dst + 1]
    lid = mo.blocks.lid[K - 1]
    dst_lid = mo.blocks.dst_lid[K - 1]
    gen = torch.Generator().manual_seed(17)
    W = (torch.randn(2 * cfg.d, SAGE_D_OUT, generator=gen) / np.sqrt(2 * cfg.d)).to(dev)
    b = torch.randn(SAGE_D_OUT, generator=gen).to(dev)
    agg = torch.empty(n_dst, cfg.ld, dtype=torch.float32, device=dev)
    out = torch.empty(n_dst, SAGE_D_OUT, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def layer():
        gm.gnn_sage_layer(indptr, lid, dst_lid, mo.x, cfg.d, W, b, True, agg, out,
                          d_status=status)

    def mean():
        gm.gnn_mean_aggregate(indptr, lid, mo.x, cfg.d, agg)

    def update():
        gm.gnn_sage_update(dst_lid, mo.x, cfg.d, agg, W, b, True, out, n_dst=n_dst,
                           d_status=status)

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_layer, t_mean, t_upd = timed(layer), timed(mean), timed(update)
    if int(status.item()) != gm.GNN_OK:
        raise RuntimeError("GraphSAGE layer: device status %d" % int(status.item()))
    flops = 2.0 * n_dst * 2 * cfg.d * SAGE_D_OUT
    upd_bytes = 4.0 * (n_dst * (2 * cfg.d + SAGE_D_OUT + 1) + 2 * cfg.d * SAGE_D_OUT + SAGE_D_OUT)
    tf = flops / (t_upd * 1e-3) / 1e12
    return {"block": f"outermost block of one batch ({n_dst} destinations, {n_edges} edges), "
                     f"X as its source rows",
            "d": cfg.d, "d_out": SAGE_D_OUT, "dtype": "fp32", "relu": True,
            "layer_ms": t_layer, "mean_ms": t_mean, "update_ms": t_upd,
            "update_flops": flops, "update_algorithmic_bytes": upd_bytes,
            "update_GBps": upd_bytes / (t_upd * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "kernel": "k_sage_update", "achieved": tf,
                         "peak": FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / FP32_MFMA_TFLOPS},
            "timing": f"HIP events over {reps} calls each of the layer, the mean alone and the "
                      f"UPDATE alone, on the library's stream"}


def hash_ceiling(gm, dev, reps=3):
    """Keys per second of the sampler's key hashing alone (gnn_hash_probe: SplitMix64 finalisers
    of a stepped counter on every lane of 4096 workgroups of 256), best of `reps` launches timed
    with HIP events on the current stream."""
    import torch
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    lanes, per_lane = 4096 * 256, 4096
    gm.gnn_hash_probe(1, 1 << 60, lanes, per_lane, cnt)     # warm-up
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gm.gnn_hash_probe(2, 1 << 60, lanes, per_lane, cnt)
        e1.record()
        e1.synchronize()
        best = max(best, lanes * per_lane / (e0.elapsed_time(e1) / 1e3))
    return best


def host_link(gm, table, dev):
    """Host -> device bandwidth: the best of 5 hipMemcpyAsync copies of 1 GiB from pinned host
    memory (B_link), and the best of 5 zero-copy streaming reads of the same bytes by a kernel."""
    import torch

    n = (1 << 30) // 4
    src = table.view(-1)[:n]
    dst = torch.empty(n, dtype=torch.float32, device=dev)
    best_copy, best_zc = 0.0, 0.0
    for _ in range(5):
        for kind in ("copy", "zero_copy"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if kind == "copy":
                dst.copy_(src, non_blocking=True)
            else:
                gm.gnn_copy_probe_host(src, dst)
            e1.record()
            e1.synchronize()
            gbps = n * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9
            if kind == "copy":
                best_copy = max(best_copy, gbps)
            else:
                best_zc = max(best_zc, gbps)
    del dst
    return {"B_link_GBps": best_copy, "zero_copy_read_GBps": best_zc}


def cpu_info():
    """The host's CPU model (lscpu, else /proc/cpuinfo) and its logical CPU count."""
    import platform
    import subprocess
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None and os.path.exists("/proc/cpuinfo"):
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    return {"cpu_model": model or platform.processor() or "unknown", "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def system_fingerprint(dev):
    """The GPU (name, architecture, compute units, memory, LDS per workgroup), the ROCm and
    PyTorch versions and the host CPU of the run."""
    import torch
    p = torch.cuda.get_device_properties(dev)
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(path):
            rocm = open(path).read().strip()
            break
    return dict({"gpu": p.name, "arch": getattr(p, "gcnArchName", None),
                 "compute_units": p.multi_processor_count, "hbm_bytes": p.total_memory,
                 "lds_per_workgroup": getattr(p, "shared_memory_per_block", None),
                 "rocm": rocm, "torch": torch.__version__, "hip": torch.version.hip},
                **cpu_info())


def cpu_baseline(cfg, graph, table, step, budget_s, gpu_value):
    """The oracle (single-threaded C) on the first super-batches of the same epoch, until budget_s
    of CPU work has been spent; checks its results against the GPU path's on those batches: every
    block array and X bit for bit, every h within 1e-5 * max|X|."""
    import numpy as np
    import torch

    import oracle

    indptr = graph.indptr.cpu().numpy()
    indices = graph.indices.cpu().numpy()
    x = table.cpu().numpy()
    K = len(cfg.fanouts)
    spent, edges, batches, parity, st = 0.0, 0, 0, True, 0
    mismatch = []
    while spent < budget_s and batches < 64:
        s, mine, sb_seeds = step(st)
        torch.cuda.synchronize()
        st += 1
        seed64 = oracle.batch_seed(cfg.rng_seed, s)
        sb_h = sb_seeds.cpu().numpy()
        off = 0
        for b, n, got in mine:
            seeds = sb_h[off:off + n]
            off += n
            if spent >= budget_s and batches > 0:
                break
            t0 = time.perf_counter()
            ref = oracle.minibatch(indptr, indices, x, seeds, cfg.fanouts, seed64, d=cfg.d)
            spent += time.perf_counter() - t0
            edges += sum(len(bl.gid) for bl in ref.blocks)
            batches += 1
            host = got.blocks.host()
            for l in range(K):
                rb = ref.blocks[l]
                for name, g_arr, r_arr in (("indptr", host[l][0], rb.indptr),
                                           ("gid", host[l][1], rb.gid), ("lid", host[l][2], rb.lid),
                                           ("dst_lid", host[l][3], rb.dst_lid),
                                           ("nodes", host[l][4], rb.nodes)):
                    if not np.array_equal(g_arr, r_arr):
                        mismatch.append(f"batch {b} hop {l + 1} {name}")
            nv = len(ref.blocks[-1].nodes)
            xg = np.ascontiguousarray(got.x[:nv, :cfg.d].cpu().numpy())
            if not np.array_equal(xg.view(np.uint32), ref.x.view(np.uint32)):
                mismatch.append(f"batch {b} X")
            tol = 1e-5 * float(np.abs(ref.x).max()) if ref.x.size else 0.0
            for l in range(K):
                rows = ref.h[l].shape[0]
                if rows == 0:
                    continue
                err = float(np.abs(got.h[l][:rows, :cfg.d].cpu().numpy().astype(np.float64)
                                   - ref.h[l]).max())
                if err > tol:
                    mismatch.append(f"batch {b} h_{l} err {err:.3g} > {tol:.3g}")
    parity = not mismatch
    value = edges / spent
    return dict({"value": value, "unit": "sampled edges/s", "cores": 1, "kind": "oracle",
                 "sample": f"the first {batches} mini-batches of the epoch (same seeds and batch "
                           f"seed as the GPU run), whole path: sampling, relabel, gather, mean; "
                           f"{spent:.1f} s single-threaded",
                 "gpu_over_cpu": gpu_value / value, "parity_on_sample": parity,
                 "parity_checked": "every block array (indptr, gid, lid, dst_lid, V_l) and X bit "
                                   "for bit, every h_l within 1e-5 * max|X|",
                 "parity_mismatches": mismatch[:10]}, **cpu_info())


if __name__ == "__main__":
    main()
