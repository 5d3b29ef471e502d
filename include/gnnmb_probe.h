/*
 * gnnmb_probe.h -- measurement helper of libgnnmb.so (not part of the mini-batch path).
 *
 * gnn_copy_probe copies `bytes` bytes (a multiple of 16, both pointers 16-byte aligned, device
 * memory) from src to dst with a plain streaming kernel, k_copy_probe.  Its hardware counters
 * (bytes fetched from and written to memory) for a copy of known size calibrate the counter
 * readings of the other kernels.  Enqueues on `stream` and returns; GNN_ERR_INVALID_ARG on a bad
 * size or alignment.
 *
 * gnn_copy_probe_host runs the same kernel on a source in pinned (page-locked, mapped) host
 * memory, read in place over the host link: the streaming ceiling of zero-copy reads, beside
 * which the feature gather's misses to a host-resident table are measured.  host_src must come
 * from hipHostMalloc (or torch's pin_memory); GNN_ERR_HIP if it has no device mapping.
 *
 * gnn_hash_probe: `lanes` work-items (a multiple of 256) each evaluate `per_lane` (even) sampling
 * keys, SplitMix64 mix64 of a stepped counter as in the sampler's candidate loop, and add the
 * number of keys <= tau to *d_count (device uint64).  Keys per second of this launch are the
 * measured ceiling of the hashing that the sampler does for every position of a long row.
 */
#ifndef GNNMB_PROBE_H
#define GNNMB_PROBE_H

#include "gnnmb.h"

#ifdef __cplusplus
extern "C" {
#endif

gnn_status gnn_copy_probe(const void *src, void *dst, size_t bytes, gnn_stream stream);
gnn_status gnn_copy_probe_host(const void *host_src, void *dst, size_t bytes, gnn_stream stream);
gnn_status gnn_hash_probe(uint64_t seed, uint64_t tau, int64_t lanes, int64_t per_lane,
                          unsigned long long *d_count, gnn_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* GNNMB_PROBE_H */
