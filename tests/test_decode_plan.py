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
