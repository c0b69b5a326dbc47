"""Zigzag partition: the host-side plan of sub-block products (no GPU).

The pages' fix for the causal load imbalance ("Ring Attention Paper Breakdown:
Blockwise Distributed Transformers for Near-Infinite Context", section 5;
"Ring Attention：把超长序列沿设备环流动", section "Causal Attention 让环不再完全对称"):
cut the sequence into 2P pieces and give rank i pieces i and 2P-1-i.  These
tests pin the plan that ZigzagRing follows against what the partition implies:
every (query piece, key piece) pair with the key piece not after the query
piece is computed exactly once over all ranks, and every rank has the same
work.
"""
import pytest

from ring_attention_block_amd import _lib
from ring_attention_block_amd.ring import ring_order, zigzag_blocks, zigzag_plan

FULL, DIAG, SKIP = _lib.RA_CASE_FULL, _lib.RA_CASE_DIAG, _lib.RA_CASE_SKIP


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16])
def test_every_causal_pair_exactly_once(P):
    seen = {}
    for rank in range(P):
        plan = zigzag_plan(rank, P, True)
        assert [j for j, _ in plan] == ring_order(rank, P)
        mine = zigzag_blocks(rank, P)
        for j, prods in plan:
            theirs = zigzag_blocks(j, P)
            assert sorted((a, b) for a, b, _ in prods) == [(0, 0), (0, 1), (1, 0), (1, 1)]
            for a, b, case in prods:
                qb, kb = mine[a], theirs[b]
                want = SKIP if kb > qb else DIAG if kb == qb else FULL
                assert case == want, (P, rank, j, a, b)
                if case != SKIP:
                    assert (qb, kb) not in seen
                    seen[(qb, kb)] = rank
    # all pairs kb <= qb over the 2P pieces, and the query piece's owner computed it
    assert sorted(seen) == [(q, k) for q in range(2 * P) for k in range(q + 1)]
    for (qb, _), rank in seen.items():
        assert qb in zigzag_blocks(rank, P)


@pytest.mark.parametrize("P", [1, 2, 4, 8, 16, 64])
def test_equal_work_per_rank(P):
    rows = 1000   # tokens per piece
    for rank in range(P):
        cases = [c for _, prods in zigzag_plan(rank, P, True) for _, _, c in prods]
        assert cases.count(FULL) == 2 * P - 1 and cases.count(DIAG) == 2
        pairs = cases.count(FULL) * rows * rows + cases.count(DIAG) * rows * (rows + 1) // 2
        # the rank's share of all N(N+1)/2 causal pairs of N = 2P * rows tokens
        n = 2 * P * rows
        assert pairs * P == n * (n + 1) // 2


@pytest.mark.parametrize("P", [1, 3, 8])
def test_non_causal_is_all_full(P):
    for rank in range(P):
        for _, prods in zigzag_plan(rank, P, False):
            assert [c for _, _, c in prods] == [FULL] * 4
