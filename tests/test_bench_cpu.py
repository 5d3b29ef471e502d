"""The benchmark's host-side logic (CPU only): the one-GPU guard, the algorithmic byte model and
the names of the kernel instances it reports."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert "one GPU" in json.loads(line)["error"]


def test_algorithmic_bytes_by_hand():
    # two hops: 3 seeds; block 1: 5 edges, |V_1| = 6; block 2: 9 edges, |V_2| = 11; d = 2
    gather, mean, E, V = bench.algorithmic_bytes([5, 6, 9, 11], 3, 2, 2)
    assert (E, V) == ([5, 9], [6, 11])
    assert gather == 11 * (4 + 2 * 2 * 4)                   # id + row read + row write
    # block 1: sources V_1 rows, 5 lids, 4 indptr entries, 3 output rows
    assert mean[0] == 6 * 8 + 5 * 4 + 4 * 4 + 3 * 8
    # block 2: sources V_2 rows, 9 lids, 7 indptr entries, 6 output rows
    assert mean[1] == 11 * 8 + 9 * 4 + 7 * 4 + 6 * 8


def test_kernel_instances_follow_row_shape():
    assert bench.kernel_instance("gather", 602, 604, True) == "k_gather_batch<64, 3, 8>"
    assert bench.kernel_instance("mean", 602, 604, True) == "k_mean_v5<64, 3, 2>"
    assert bench.kernel_instance("gather", 100, 100, True) == "k_gather_batch<32, 1, 4>"
    assert bench.kernel_instance("gather", 64, 64, False) == "k_gather_rows<16, 1, 4>"
    assert bench.kernel_instance("gather", 13, 13, True) == "k_gather<1, 4>"   # unaligned rows
    assert bench.kernel_instance("gather", 602, 604, True, True) == "k_gather_rows<64, 3, 8, true>"


def test_union_gather_choice():
    import synth
    dense, mid, billion = (synth.CONFIGS[n] for n in ("dense", "mid", "billion"))
    assert bench.union_gather(dense, "auto", 8)
    assert not bench.union_gather(dense, "auto", 1)           # one batch: nothing to share
    assert not bench.union_gather(dense, "interleaved", 8)
    assert not bench.union_gather(mid, "auto", 8)             # 100-float rows
    assert not bench.union_gather(billion, "auto", 8)         # host-resident table


def test_sampler_ceiling_model():
    # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz over 19 instructions per key (reported beside the
    # ceiling the benchmark measures with the hash probe)
    assert abs(bench.KEYS_PEAK_MODEL - 2.07e12) / 2.07e12 < 0.01


def test_stage_percentiles():
    import numpy as np
    st = np.array([[i, 2 * i, 0, 1, 0.5 * i] for i in range(1, 11)], dtype=np.float64)
    p = bench.percentiles(st)
    assert p["sample_relabel"]["median"] == 5.5
    assert p["gather"]["p10"] == np.percentile(2 * np.arange(1, 11), 10)
    assert p["step"]["p90"] == np.percentile(3 * np.arange(1, 11) + 1, 90)


def test_cpu_info_names_the_host():
    info = bench.cpu_info()
    assert info["nproc"] >= 1 and info["cpu_model"]


def test_super_batch_size_default():
    import synth
    assert bench.super_batch_size(synth.CONFIGS["mid"], 0) == 8      # fixed by the workload
    assert bench.super_batch_size(synth.CONFIGS["dense"], 0) == bench.DEFAULT_GROUP
    assert bench.super_batch_size(synth.CONFIGS["billion"], 0) == bench.DEFAULT_GROUP
    assert bench.super_batch_size(synth.CONFIGS["mid"], 4) == 4      # asked for
