"""Decode reduction tree (host logic, no GPU): every shard's state reaches state
0 exactly once, and the merges of one level touch disjoint states."""
import pytest

from ring_attention_block_amd.decode import merge_tree


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 13, 64])
def test_merge_tree_reduces_every_shard_once(n):
    holds = {p: {p} for p in range(n)}          # shards folded into each state
    for level in merge_tree(n):
        touched = [p for pair in level for p in pair]
        assert len(touched) == len(set(touched))  # independent merges within a level
        for dst, src in level:
            assert holds[src] and not (holds[dst] & holds[src])
            holds[dst] |= holds.pop(src)
    assert holds == {0: set(range(n))}
    assert len(merge_tree(n)) == (n - 1).bit_length()


def test_splits_for_fills_two_workgroups_per_unit():
    from ring_attention_block_amd.decode import splits_for
    # 8 shards x 32 heads: 256 workgroups alone, two chunks per shard give 512
    assert splits_for(8, 32, 4096, 1) == 2
    assert splits_for(8, 32, 4096, 16) == 2
    assert splits_for(8, 32, 4096, 32) == 2
    assert splits_for(8, 32, 4096, 33) == 1      # longer query blocks are not split
    assert splits_for(8, 32, 4096, 256) == 1
    assert splits_for(8, 64, 4096, 1) == 1       # 512 workgroups already
    assert splits_for(1, 1, 4096, 1) == 64       # 512 would need chunks of 8 keys: stops at 64 keys
    assert splits_for(4, 32, 4096, 1) == 4
    assert splits_for(8, 32, 3000, 1) == 2       # smallest divisor giving enough
    assert splits_for(8, 32, 127, 1) == 1        # no divisor leaves chunks of >= 64 keys
    for shards, heads, rows in [(8, 32, 4096), (3, 5, 960), (2, 7, 1000), (16, 2, 64)]:
        s = splits_for(shards, heads, rows, 1)
        assert rows % s == 0 and (s == 1 or rows // s >= 64)
    with pytest.raises(ValueError):
        splits_for(0, 32, 4096, 1)
