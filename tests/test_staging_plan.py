"""Staging mode of a forward ring (no GPU): ring.staging_for, the choice bench.py
makes with --staging auto between copy kernels on a side stream ordered by events
("side") and copies carried by the step launches on the compute stream alone
("fused", ra_step_staged).  Both give bit-identical rings (GPU tests); the choice
is a matter of speed: long steps hide a copy kernel beside them, short steps and
visits that fold nothing do better without the events."""
from ring_attention_block_amd.ring import staging_for


def test_staging_choice_for_the_workloads():
    # 32 heads x 4096 rows, d 128: 275 GFLOP per full step, rank 7 skips nothing
    assert staging_for(32, 4096, 4096, 128, skipped_visits=0) == "side"
    # ranks 0 and 3 of the same ring skip 7 and 4 visits
    assert staging_for(32, 4096, 4096, 128, skipped_visits=7) == "fused"
    assert staging_for(32, 4096, 4096, 128, skipped_visits=4) == "fused"
    # stress ring: 8 heads x 2048 rows, each block as two key ranges (state batch 2)
    assert staging_for(2 * 8, 2048, 1024, 128, skipped_visits=0) == "fused"
    # zigzag piece products: 32 heads x 2048 x 2048, d 128 (69 GFLOP)
    assert staging_for(32, 2048, 2048, 128, skipped_visits=0) == "fused"
    # long-share d 64 (1.1 TFLOP) and million-token d 128 (1.1 TFLOP) steps
    assert staging_for(16, 16384, 16384, 64, skipped_visits=0) == "side"
    assert staging_for(8, 16384, 16384, 128, skipped_visits=0) == "side"


def test_staging_threshold():
    # exactly at the threshold: side; just below: fused
    rows = 4096
    heads_at = int(100e9 / (4 * 128 * rows * rows)) + 1
    assert staging_for(heads_at, rows, rows, 128, 0) == "side"
    assert staging_for(1, rows, rows, 128, 0) == "fused"
    assert staging_for(32, 4096, 4096, 128, 0, min_step_gflop=300.0) == "fused"
