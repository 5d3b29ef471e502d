"""The partitioned GPU R-MAT builder gives the same graph as the chunked torch builder.

The draw kernel regenerates the draws per destination range; forcing many ranges, and a first
draw budget too small for the requested edge count (so the budget grows and the draws are
redone), must not change a single edge."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,e,parts_draws,draws", [
    (10_000, 160_000, 1 << 16, None),       # tiny workload's size, ~20 ranges
    (100_000, 2_000_000, 1 << 18, None),     # ~12 ranges
    (64, 3_000, 1 << 12, 3_100),             # dense: heavy duplication, budget regrown
    (1_000, 20_000, 1 << 30, 20_000),        # one range, budget regrown
])
def test_partitioned_equals_chunked(n, e, parts_draws, draws):
    a, b, c = 0.57, 0.19, 0.19
    ref = synth.rmat_csr(n, e, a, b, c, 77, torch.int64, "cuda")
    got = synth.rmat_csr_partitioned(n, e, a, b, c, 77, torch.int64, "cuda",
                                     draws_per_part=parts_draws, draws=draws)
    assert torch.equal(ref.indptr, got.indptr)
    assert torch.equal(ref.indices, got.indices)


def test_tiny_config_both_builders():
    cfg = synth.CONFIGS["tiny"]
    ref = synth.build_graph(cfg, device="cpu")
    got = synth.rmat_csr_partitioned(cfg.num_nodes, cfg.num_edges, *cfg.rmat, cfg.rng_seed,
                                     torch.int32, "cuda", draws_per_part=1 << 17)
    assert torch.equal(ref.indptr, got.indptr.cpu())
    assert torch.equal(ref.indices, got.indices.cpu())
