"""CPU checks of bench.py's accounting: the algorithmic bytes its roofline
figures divide by, its refusal of more than one GPU, and which workload its counter
record belongs to."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def shape(lens, K=1):
    return dict(seq_lens=np.asarray(lens, np.int32), rows_per_seq=K, index_dim=128,
                index_heads=32, num_heads=64, latent_dim=512, top_k=2048, page_size=64)


def test_long_workload_bytes():
    ab = bench.algorithmic_bytes(shape([131072] * 8))
    keys = 8 * 131072 * 128 * 2                 # every visible key once
    qw = 8 * 32 * (128 * 2 + 4)                  # indexer query and weights per row
    gather = 8 * 2048 * 512                      # selected FP8 latent rows
    qo = 8 * 64 * 512 * 2 * 2                    # bf16 query in, bf16 output out
    bt = 8 * 2048 * 4                            # one block-table entry per selected token, at most
    assert ab["index"] == keys + qw == 268_502_016
    assert ab["attend"] == gather + qo + bt
    assert ab["total"] == 278_004_736


def test_rows_of_a_sequence_share_its_keys():
    # four verify rows of one sequence read that sequence's keys once, up to
    # the longest row; each row still gathers its own selection
    one = bench.algorithmic_bytes(shape([16388], K=1))
    four = bench.algorithmic_bytes(shape([16385, 16386, 16387, 16388], K=4))
    assert four["index"] - 4 * 32 * 260 == one["index"] - 32 * 260
    assert four["attend"] == 4 * one["attend"]


def test_short_rows_count_only_what_they_select():
    # a row shorter than top_k selects (and gathers) every token, no more
    ab = bench.algorithmic_bytes(shape([1000]))
    assert ab["attend"] == 1000 * 512 + 64 * 512 * 4 + (1000 + 63) // 64 * 4


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_traffic_record_is_only_reported_for_its_own_workload():
    rec = json.load(open(bench.TRAFFIC_FILE))
    if rec.get("kernel_sha") != bench.kernel_sha():
        pytest.skip("the committed counter record predates the current index kernel")
    assert bench.load_traffic("long") == rec["bytes_per_launch"]
    for w in ("kverify", "batched", "single", "rowgroup", "tiny"):
        assert bench.load_traffic(w) is None
