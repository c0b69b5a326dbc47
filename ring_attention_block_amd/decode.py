"""Decode / short query block against a sharded key/value cache, on one GPU.

The pages' decoding pattern ("Ring Attention：把超长序列沿设备环流动", section
"训练与推理的适用方式不同"): rather than passing key/value blocks around the ring
for one new query, the short query block (the newest tokens) is broadcast to
the ranks that hold the key/value shards; each rank folds it against its own
shard into a partial softmax state, and a global online-softmax reduction
combines the partial states.  The reduction is the merge of the aicassindra
architecture article (section "The architecture: every piece explained"),
whose identity is the empty state, so any tree of merges gives the same result
up to rounding.

The shards hold keys that every new token may see (the history before the
block; a single new token's own key may be the last one), so the local folds
run without the causal mask; that is what lets ra_step take a key/value block
of another length than the query block.  ShardedDecode runs the P ranks as P
streams of one GPU: the local folds run concurrently, and a binary tree of
ra_lse_merge calls reduces the P states into state 0 on the compute stream,
which then finalizes.  ChunkedDecode folds every shard in one launch and
reduces and finalizes in a second one (ra_merge_finalize).
"""
from __future__ import annotations

from typing import Sequence

import torch

from . import _lib
from .hip_events import Event


def merge_tree(shards: int) -> list:
    """Levels of a binary reduction of `shards` states into state 0: each level
    is a list of (dst, src) pairs whose merges are independent."""
    levels, stride = [], 1
    while stride < shards:
        levels.append([(p, p + stride) for p in range(0, shards, 2 * stride) if p + stride < shards])
        stride *= 2
    return levels


class ShardedDecode:
    """Reusable states, streams and events for decoding against `shards` shards.

    q_shape: [batch, heads, rows, head_dim] of the query block.
    """

    def __init__(self, q_shape, shards: int, device="cuda", compute_stream=None):
        b, h, rows, d = q_shape
        self.shards = shards
        self.states = [_lib.State(b, h, rows, d, device=device) for _ in range(shards)]
        self.compute = compute_stream if compute_stream is not None else torch.cuda.current_stream()
        self.streams = [torch.cuda.Stream(device=device) for _ in range(shards)]
        self.ev_start = Event()
        self.ev_done = [Event() for _ in range(shards)]

    def run(self, q: torch.Tensor, kv: Sequence[tuple], scale: float, out_dtype=torch.float32,
            o_out=None, lse_out=None):
        """kv[p] = (K_p, V_p), [batch, heads, kv_rows_p, head_dim] each.  Returns
        the finalized (O, LSE) of q against the concatenation of all shards."""
        if len(kv) != self.shards:
            raise ValueError(f"expected {self.shards} shards, got {len(kv)}")
        # The local folds start after everything queued on the compute stream.
        self.ev_start.record(self.compute)
        for p, (k, v) in enumerate(kv):
            s = self.streams[p]
            self.ev_start.wait(s)
            # The local fold starts from the empty state (init fused into the step).
            _lib.step(self.states[p], q, k, v, 0, 0, 1, False, scale, s, flags=_lib.RA_STEP_FRESH)
            self.ev_done[p].record(s)
        for p in range(self.shards):
            self.ev_done[p].wait(self.compute)
        for level in merge_tree(self.shards):
            for dst, src in level:
                _lib.lse_merge(self.states[dst], self.states[src], self.compute)
        return _lib.finalize(self.states[0], out_dtype, self.compute, o_out=o_out,
                             lse_out=lse_out)


def splits_for(shards: int, heads: int, shard_rows: int, query_rows: int,
               compute_units: int = 256) -> int:
    """Chunks per shard for ChunkedDecode.  A query block of at most 32 rows
    (one wavefront's rows: the fold is a pure stream of the cache) takes the
    fewest chunks that give the fold launch two workgroups per compute unit
    (shards * splits * heads >= 2 * compute_units), among the divisors of the
    shard length that leave chunks of at least 64 keys; longer query blocks,
    and shards that already give enough workgroups, take 1.  Two workgroups per
    unit keep twice the key/value tiles in flight; more chunks add partial
    states to reduce.  Measured at 8 shards of 4096 keys and 32 heads (decode
    step, ms, 1 chunk per shard against 2): 0.1058 / 0.0993 at 1 new row,
    0.1063 / 0.1029 at 16, 0.1137 / 0.1130 at 64, 0.1790 / 0.1971 at 256;
    4 and 8 chunks per shard were slower than 2 at 1 and 16 rows."""
    if shards < 1 or heads < 1 or shard_rows < 1 or query_rows < 1:
        raise ValueError("shards, heads, shard_rows and query_rows must be positive")
    s = 1
    if query_rows > 32:
        return s
    while shards * s * heads < 2 * compute_units:
        nxt = next((x for x in range(s + 1, shard_rows + 1)
                    if shard_rows % x == 0 and shard_rows // x >= 64), None)
        if nxt is None:
            break
        s = nxt
    return s


class ChunkedDecode:
    """Decode with the key/value cache laid out as chunks along the batch axis.

    The cache (all shards) is held as K, V of shape [chunks, heads, chunk_rows,
    head_dim]: chunk c is a contiguous [heads, chunk_rows, head_dim] slab.  One
    ra_step launch folds the query block [1, heads, rows, head_dim] against all
    chunks at once (RA_STEP_Q_BROADCAST: every batch entry of the state reads
    the one query block; batch = chunks, so every chunk and head has its own
    workgroups); one ra_merge_finalize launch then reduces
    the chunks' partial states (the merge is associative and commutative up to
    rounding) and writes the finalized output.  Two launches on one stream,
    with no cross-stream synchronisation.
    """

    def __init__(self, q_shape, chunks: int, device="cuda", compute_stream=None):
        b, h, rows, d = q_shape
        if b != 1:
            raise ValueError("the query block must have batch 1")
        if chunks < 1:
            raise ValueError(f"chunks={chunks} must be positive")
        self.chunks = chunks
        self.q_shape = tuple(q_shape)
        self.state = _lib.State(chunks, h, rows, d, device=device)
        self.compute = compute_stream if compute_stream is not None else torch.cuda.current_stream()

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
            out_dtype=torch.float32, o_out=None, lse_out=None, start=None, stop=None):
        """k, v: [chunks, heads, chunk_rows, head_dim].  Returns the finalized
        (O, LSE) of q against all chunks.  start, stop: optional timing events
        bound to the fold's step kernel (ra_step_timed)."""
        n = self.chunks
        if tuple(k.shape[:2]) != (n, self.q_shape[1]) or k.shape != v.shape:
            raise ValueError(f"k, v must be [{n}, {self.q_shape[1]}, chunk_rows, d]")
        if tuple(q.shape) != self.q_shape:
            raise ValueError(f"q must be {self.q_shape}")
        _lib.step(self.state, q, k, v, 0, 0, 1, False, scale, self.compute,
                  flags=_lib.RA_STEP_FRESH | _lib.RA_STEP_Q_BROADCAST, start=start, stop=stop)
        return _lib.merge_finalize(self.state, n, out_dtype, self.compute, o_out=o_out,
                                   lse_out=lse_out)
