"""Host logic of the hot-row ranking (count desc, degree desc, id asc); runs on the CPU."""
import torch

from graph_mini_pipeline_amd.hotness import rank_adjacency, rank_rows


def test_rank_order_and_ties():
    counts = torch.tensor([0, 3, 3, 1, 0, 3], dtype=torch.int32)
    deg = torch.tensor([9, 2, 5, 7, 1, 5])
    # count 3: ids 1 (deg 2), 2 (deg 5), 5 (deg 5) -> 2, 5 (tie on degree: id asc), 1
    assert rank_rows(counts, deg, 6).tolist() == [2, 5, 1, 3, 0, 4]
    assert rank_rows(counts, deg, 2).tolist() == [2, 5]


def test_rank_all_zero_counts_is_degree_order():
    g = torch.Generator().manual_seed(5)
    deg = torch.randint(0, 1000, (5000,), generator=g)
    counts = torch.zeros(5000, dtype=torch.int32)
    got = rank_rows(counts, deg, 5000)
    ref = sorted(range(5000), key=lambda v: (-int(deg[v]), v))
    assert got.tolist() == ref


def test_rank_is_a_permutation_prefix():
    g = torch.Generator().manual_seed(6)
    counts = torch.randint(0, 65, (20000,), generator=g, dtype=torch.int32)
    deg = torch.randint(0, 1 << 20, (20000,), generator=g)
    got = rank_rows(counts, deg, 777)
    ref = sorted(range(20000), key=lambda v: (-int(counts[v]), -int(deg[v]), v))[:777]
    assert got.tolist() == ref


def test_rank_rows_degree_ascending():
    # equal counts: the short rows first when asked (the adjacency cache's order)
    counts = torch.tensor([2, 5, 5, 0, 5], dtype=torch.int32)
    degree = torch.tensor([9, 7, 3, 1, 7], dtype=torch.int64)
    assert rank_rows(counts, degree, 5, degree_desc=False).tolist() == [2, 1, 4, 0, 3]
    assert rank_rows(counts, degree, 5).tolist() == [1, 4, 2, 0, 3]


def test_rank_adjacency_by_saved_reads_per_cached_id():
    # fanouts [2, 3]; node: degree, frontier counts at levels 0 and 1
    #   0: deg 100, counts (5, 5): saved 5*2 + 5*3 = 25, per id 0.25
    #   1: deg 2,   counts (1, 0): saved 2,              per id 1.0
    #   2: deg 4,   counts (0, 2): saved 6,              per id 1.5
    #   3: deg 0,   counts (3, 3): saves nothing (an empty row)
    #   4: deg 3,   counts (0, 0): never a frontier node
    #   5: deg 6,   counts (2, 1): saved 4 + 3 = 7,      per id 7/6
    #   6: deg 1,   counts (0, 1): saved 1,              per id 1.0 (ties with node 1: id order)
    degree = torch.tensor([100, 2, 4, 0, 3, 6, 1])
    counts = torch.tensor([[5, 1, 0, 3, 0, 2, 0],
                           [5, 0, 2, 3, 0, 1, 1]], dtype=torch.int32)
    assert rank_adjacency(counts, degree, [2, 3]).tolist() == [2, 5, 1, 6, 0]

    # with out-degrees, the rows the pre-sampling never reached follow (largest fanout 3): node 4
    # (deg 3, listed by 5 rows: 5 * 3 / 3) before node 7 (deg 8, listed by 6 rows: 6 * 3 / 8);
    # node 8 is in no row, node 3's row is empty
    degree = torch.tensor([100, 2, 4, 0, 3, 6, 1, 8, 2])
    counts = torch.tensor([[5, 1, 0, 3, 0, 2, 0, 0, 0],
                           [5, 0, 2, 3, 0, 1, 1, 0, 0]], dtype=torch.int32)
    outdeg = torch.tensor([1, 1, 1, 1, 5, 1, 1, 6, 0])
    assert rank_adjacency(counts, degree, [2, 3], outdeg).tolist() == [2, 5, 1, 6, 0, 4, 7]
