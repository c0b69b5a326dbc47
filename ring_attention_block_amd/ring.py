"""Single-GPU emulation of one rank's ring.

The pages' ring ("Ring Attention Paper Breakdown: Blockwise Distributed
Transformers for Near-Infinite Context", section 2): at step s rank i computes
on key/value block j = (i - s) mod P held in buffer A while the next block is
received into buffer B on a separate stream; the buffers swap at the end of the
step.  "Ring Attention：把超长序列沿设备环流动", section "双缓冲是重叠成立的基础"
(double buffering), states the two hazards: A must not be overwritten before
the compute that reads it has finished, and B must not be read before its
transfer has finished.

Here the "receive" is a device-to-device copy (ra_stage_block) of block j from
where it sits in HBM into the free buffer, on a side stream; HIP events enforce
both hazards.  Blocks that the causal rule skips are still staged, because the
ring forwards them.  Step 0 computes on the rank's first block where it lies
(its own block, which a real rank already holds).
"""
from __future__ import annotations

from typing import Callable, Sequence

import torch

from . import _lib
from .hip_events import Event


def ring_order(rank: int, blocks: int) -> list:
    """Block visited at ring step s: (rank - s) mod blocks."""
    return [(rank - s) % blocks for s in range(blocks)]


class RingEmulator:
    """Reusable buffers, streams and events for one rank's ring.

    shape: [batch, heads, rows, head_dim] of one key (or value) block.
    """

    def __init__(self, shape, dtype, device="cuda", compute_stream=None, copy_stream=None):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.bufs = [(torch.empty(self.shape, dtype=dtype, device=device),
                      torch.empty(self.shape, dtype=dtype, device=device)) for _ in range(2)]
        self.compute = compute_stream if compute_stream is not None else torch.cuda.current_stream()
        self.copy = copy_stream if copy_stream is not None else torch.cuda.Stream(device=device)
        self.ev_ready = [Event(), Event()]
        self.ev_free = [Event(), Event()]
        self.ev_start = Event()

    def run(self, st: _lib.State, q: torch.Tensor, kv_source: Callable[[int], tuple],
            rank: int, num_blocks: int, causal: bool, scale: float,
            order: Sequence[int] | None = None, init: bool = True,
            step_timers: list | None = None, timer_events=None) -> list:
        """Fold the blocks of `order` (default: the ring order of `rank`) into st.

        kv_source(j) returns the resident (K_j, V_j) device tensors.
        step_timers, if given, receives (case, start_event, end_event) per
        launched step, recorded on the compute stream around the launch;
        timer_events, if given, is an iterator of timing events created
        beforehand (two per launched step), so that no event is created while
        work is being enqueued.  Returns the causal case of each step.
        """
        order = ring_order(rank, num_blocks) if order is None else list(order)
        comp, copy = self.compute, self.copy
        if init:
            _lib.state_init(st, comp)
        # Copies of this run start after everything already queued on the
        # compute stream (earlier runs may still read the buffers).
        self.ev_start.record(comp)
        self.ev_start.wait(copy)

        cur = kv_source(order[0])
        cur_buf = None           # index of the buffer `cur` lives in (None: source)
        free_buf = 0
        cases = []
        for s, j in enumerate(order):
            nxt_buf = None
            if s + 1 < len(order):
                nxt_buf = free_buf
                k_src, v_src = kv_source(order[s + 1])
                kb, vb = self.bufs[nxt_buf]
                _lib.stage_block(kb, k_src, copy)
                _lib.stage_block(vb, v_src, copy)
                self.ev_ready[nxt_buf].record(copy)
            if cur_buf is not None:
                self.ev_ready[cur_buf].wait(comp)
            case = _lib.step_case(rank, j, num_blocks, causal)
            if step_timers is not None and case != _lib.RA_CASE_SKIP:
                if timer_events is not None:
                    e0, e1 = next(timer_events), next(timer_events)
                else:
                    e0, e1 = Event(timing=True), Event(timing=True)
                e0.record(comp)
                _lib.step(st, q, cur[0], cur[1], rank, j, num_blocks, causal, scale, comp)
                e1.record(comp)
                step_timers.append((case, e0, e1))
            else:
                _lib.step(st, q, cur[0], cur[1], rank, j, num_blocks, causal, scale, comp)
            cases.append(case)
            if cur_buf is not None:
                self.ev_free[cur_buf].record(comp)
            if nxt_buf is not None:
                # The buffer just computed on becomes the next receive target;
                # the copy stream waits for its free event before refilling it.
                if cur_buf is not None:
                    free_buf = cur_buf
                    self.ev_free[cur_buf].wait(copy)
                else:
                    free_buf = 1 - nxt_buf
                cur, cur_buf = self.bufs[nxt_buf], nxt_buf
        return cases
