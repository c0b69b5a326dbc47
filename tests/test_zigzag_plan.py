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


def _covered(launch, h):
    """(row, key) local index pairs a launch folds, for sub-blocks of h rows:
    FULL every pair of its ranges, DIAG the lower triangle of its ranges."""
    from ring_attention_block_amd import _lib as L_
    q_lo, q_n, kv_lo, kv_n, case = launch[:5]
    rows = range(q_lo * h, (q_lo + q_n) * h)
    keys = range(kv_lo * h, (kv_lo + kv_n) * h)
    if case == L_.RA_CASE_FULL:
        return {(r, k) for r in rows for k in keys}
    assert (q_lo, q_n) == (kv_lo, kv_n)
    return {(r, k) for r in rows for k in keys if k - kv_lo * h <= r - q_lo * h}


@pytest.mark.parametrize("P", [2, 3, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_block_launches_fold_exactly_the_allowed_positions(P, causal):
    """zigzag_launches, with and without the fused-init/finalize splits, fold
    each (query, key) pair of the rank's block against every visiting block
    exactly once iff the causal mask on global positions allows it (brute
    force over positions: sub-block b holds positions [b*h, (b+1)*h))."""
    from ring_attention_block_amd.ring import zigzag_fused_launches, zigzag_launches
    h = 3
    for rank in range(P):
        mine = zigzag_blocks(rank, P)
        pos_q = [b * h + r for b in mine for r in range(h)]
        for plan in (zigzag_launches(rank, P, causal), zigzag_fused_launches(rank, P, causal)):
            assert [j for j, _ in plan] == ring_order(rank, P)
            for j, launches in plan:
                pos_k = [b * h + r for b in zigzag_blocks(j, P) for r in range(h)]
                want = {(r, k) for r in range(2 * h) for k in range(2 * h)
                        if not causal or pos_k[k] <= pos_q[r]}
                got = []
                for l in launches:
                    got.extend(_covered(l, h))
                assert len(got) == len(set(got)), (rank, j, "a pair folded twice")
                assert set(got) == want, (rank, j)


@pytest.mark.parametrize("P", [2, 3, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_fused_launches_mark_each_sub_block_once(P, causal):
    """Each query sub-block has exactly one launch that starts it (fresh) and
    one that ends it (final); a marked launch covers no sub-block for which
    it is not the first (last) launch; under the causal mask every visit but
    those holding a split is one launch."""
    from ring_attention_block_amd.ring import zigzag_fused_launches
    for rank in range(P):
        plan = zigzag_fused_launches(rank, P, causal)
        flat = [l for _, ls in plan for l in ls]
        for p in range(2):
            mine = [n for n, l in enumerate(flat) if l[0] <= p < l[0] + l[1]]
            fresh = [n for n in mine if flat[n][5]]
            final = [n for n in mine if flat[n][6]]
            assert fresh == [mine[0]] and final == [mine[-1]], (rank, p)
        assert sum(len(ls) > 1 for _, ls in plan) <= 2, rank
        if causal and rank == P - 1:
            assert all(len(ls) == 1 for _, ls in plan)


@pytest.mark.parametrize("P", [2, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_launch_pairs_counts_what_each_launch_folds(P, causal):
    """launch_pairs (bench.py's FLOP count of a zigzag launch) equals the
    number of (query, key) pairs the launch folds, and over a ring the
    rank's 1/P share of the sequence's allowed pairs."""
    from ring_attention_block_amd.ring import launch_pairs, zigzag_fused_launches, zigzag_launches
    h = 5
    n = 2 * P * h
    total = n * (n + 1) // 2 if causal else n * n
    for rank in range(P):
        for plan in (zigzag_launches(rank, P, causal), zigzag_fused_launches(rank, P, causal)):
            got = 0
            for _, launches in plan:
                for l in launches:
                    assert launch_pairs(l, h) == len(_covered(l, h)), l
                    got += launch_pairs(l, h)
            assert got * P == total, (rank, got)
