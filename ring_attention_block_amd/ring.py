"""Single-GPU emulation of one rank's ring.

The pages' ring ("Ring Attention Paper Breakdown: Blockwise Distributed
Transformers for Near-Infinite Context", section 2): at step s rank i computes
on key/value block j = (i - s) mod P held in buffer A while the next block is
received into buffer B on a separate stream; the buffers swap at the end of the
step.  "Ring Attention：把超长序列沿设备环流动", section "双缓冲是重叠成立的基础"
(double buffering), states the two hazards: A must not be overwritten before
the compute that reads it has finished, and B must not be read before its
transfer has finished.

Here the "receive" is a device-to-device copy (ra_stage_block) of the visiting
rank's tensors from where they sit in HBM into the free buffer, on a side
stream; HIP events enforce both hazards.  Blocks that the causal rule skips
are still staged, because the ring forwards them.  Step 0 computes on the
rank's own tensors where they lie (a real rank already holds them).

Two partitions of the sequence over the P ranks:
  * contiguous: rank i holds block i of P equal blocks (RingEmulator.run);
  * zigzag ("Ring Attention Paper Breakdown ...", section 5, and
    "Ring Attention：...", section "Causal Attention 让环不再完全对称"): the
    sequence is cut into 2P sub-blocks and rank i holds sub-blocks i and
    2P-1-i, so under the causal mask every rank has the same work
    (ZigzagRing).  Each visit is then up to four ra_step calls on sub-block
    pairs; ra_step's causal case test on 2P sub-block indices already gives
    the skip / diagonal / full case of each pair.

Without the causal mask, a ring whose query block is too small to occupy the
chip can fold each visiting block as key_split ranges of keys into key_split
partial states, merged once at the end (key_split_for, split_keys,
RingEmulator.run): the merge of partial online-softmax states ("RingAttention
... 10M Tokens", the architecture section; "Ring Attention Math Deep",
online-softmax identity) makes the result independent of how the keys are
grouped, up to floating-point order.
"""
from __future__ import annotations

from typing import Callable, Sequence

import torch

from . import _lib
from .hip_events import Event


def ring_order(rank: int, blocks: int) -> list:
    """Block visited at ring step s: (rank - s) mod blocks."""
    return [(rank - s) % blocks for s in range(blocks)]


def key_split_for(batch_heads: int, rows: int, kv_rows: int, causal: bool,
                  compute_units: int = 256) -> int:
    """Key ranges per visiting block for RingEmulator.run: 1 under the causal
    mask (ra_step needs equal blocks there) or when the step's grid of
    128-row query tiles already covers the compute units; otherwise the
    smallest of 2, 4 whose grid covers them, as long as each range is a whole
    number of 64-key tiles."""
    if causal:
        return 1
    tiles = batch_heads * ((rows + 127) // 128)
    s = 1
    while s < 4 and tiles * s < compute_units and kv_rows % (2 * s * 64) == 0:
        s *= 2
    return s


def staging_for(batch_heads: int, rows: int, kv_rows: int, head_dim: int, skipped_visits: int,
                min_step_gflop: float = 100.0) -> str:
    """Staging mode of a forward ring (RingEmulator's `staging`): "side" when
    every visit launches a step of at least min_step_gflop of matrix work
    (4 * head_dim * batch_heads * rows * kv_rows FLOP): there a copy kernel
    beside the step hides almost entirely and the cross-stream events cost
    little against the step; otherwise "fused" (short steps, where the events
    and the separate copy launches dominate, and visits with nothing to fold,
    whose copies then run alone on the compute stream without events)."""
    step_flop = 4.0 * head_dim * batch_heads * rows * kv_rows
    if skipped_visits == 0 and step_flop >= min_step_gflop * 1e9:
        return "side"
    return "fused"


def split_keys(t: torch.Tensor, parts: int) -> torch.Tensor:
    """[1, H, n, d] -> [parts, H, n / parts, d]: batch entry p holds keys
    p*n/parts .. (p+1)*n/parts - 1 (the layout RingEmulator.run takes with
    key_split = parts, and the part order of ra_merge_finalize)."""
    _, h, n, d = t.shape
    if t.shape[0] != 1 or n % parts:
        raise ValueError("split_keys: needs batch 1 and a row count divisible by parts")
    return t.view(1, h, parts, n // parts, d).permute(0, 2, 1, 3, 4).reshape(parts, h, n // parts, d).contiguous()


def zigzag_blocks(rank: int, ranks: int) -> tuple:
    """The two sub-blocks (of 2*ranks) that `rank` holds under the zigzag partition."""
    return (rank, 2 * ranks - 1 - rank)


def zigzag_plan(rank: int, ranks: int, causal: bool) -> list:
    """Per ring step: (visiting rank j, [(a, b, case)]) for the products of the
    rank's query sub-block a (0, 1) with the visiting key/value sub-block b
    (0, 1); case is ra_step's causal case over 2*ranks sub-blocks (skipped
    pairs are listed too)."""
    mine = zigzag_blocks(rank, ranks)
    plan = []
    for j in ring_order(rank, ranks):
        theirs = zigzag_blocks(j, ranks)
        prods = [(a, b, _lib.step_case(mine[a], theirs[b], 2 * ranks, causal))
                 for a in range(2) for b in range(2)]
        plan.append((j, prods))
    return plan


class RingEmulator:
    """Reusable buffers, streams and events for one rank's ring.

    shape: [batch, heads, rows, head_dim] of one staged tensor;
    tensors_per_visit: tensors staged per visiting rank (K, V for the
    contiguous partition; K and V of two sub-blocks for zigzag);
    extra_specs: (shape, dtype) of further tensors staged with them (the
    travelling dK, dV accumulators of the backward);
    staging: "side" (copy kernels on a side stream, events between the
    streams) or "fused" (the copies ride in the step launches, ra_step_staged;
    forward rings only).
    """

    def __init__(self, shape, dtype, device="cuda", compute_stream=None, copy_stream=None,
                 tensors_per_visit: int = 2, extra_specs=(), staging: str = "side"):
        if staging not in ("side", "fused"):
            raise ValueError(f"staging must be 'side' or 'fused', got {staging!r}")
        # staging "side": each block is staged by a copy kernel on the copy
        # stream, ordered against the steps by events.  "fused": the copies of
        # the next visit ride in the current visit's step launches
        # (ra_step_staged), on the compute stream alone, with no events.
        self.staging = staging
        self.pending = []            # fused: (dst, src) copies not yet given to a launch
        self.copies_per_launch = 2   # fused: copies one step launch takes at most
        self.shape = tuple(shape)
        self.dtype = dtype
        specs = [(self.shape, dtype)] * tensors_per_visit + [(tuple(sh), dt) for sh, dt in extra_specs]
        self.bufs = [tuple(torch.empty(sh, dtype=dt, device=device) for sh, dt in specs)
                     for _ in range(2)]
        self.compute = compute_stream if compute_stream is not None else torch.cuda.current_stream()
        self.copy = copy_stream if copy_stream is not None else torch.cuda.Stream(device=device)
        self.ev_ready = [Event(), Event()]
        self.ev_free = [Event(), Event()]
        self.ev_start = Event()
        self.last_stop = None
        # free_hook(tensors, copy_stream), if set, is enqueued on the copy
        # stream each time a receive buffer is released: after the stream has
        # waited for the buffer's free event (and after the drain), before the
        # next block is staged into it.  Tests poison released buffers with it.
        self.free_hook = None

    def visit(self, order: Sequence[int], source: Callable[[int], tuple],
              fold: Callable[[int, int, tuple], None], drain=None, busy=None) -> None:
        """The staging protocol: for each step s, fold(s, j, tensors) enqueues
        the compute on visiting rank j = order[s] on the compute stream while
        the tensors of order[s+1] are staged into the free buffer.

        drain(j, tensors, stream), if given, is enqueued on the copy stream
        once the compute on a staged buffer has finished and before the buffer
        is refilled: the send of what the step updated (the backward's dK, dV)
        to the next rank.  The compute stream waits for the last drain.

        busy(s), if given, says whether step s launches any compute; the
        staging that overlaps a step that does not (a skipped causal block)
        runs alone and takes the whole chip (ra_stage_block_ex)."""
        if self.staging == "fused":
            self._visit_fused(order, source, fold, drain, busy)
            return
        comp, copy = self.compute, self.copy
        # Copies of this run start after everything already queued on the
        # compute stream (earlier runs may still read the buffers).
        self.ev_start.record(comp)
        self.ev_start.wait(copy)
        cur = source(order[0])
        cur_buf = None           # index of the buffer `cur` lives in (None: source)
        free_buf = 0
        for s, j in enumerate(order):
            nxt_buf = None
            if s + 1 < len(order):
                nxt_buf = free_buf
                alone = busy is not None and not busy(s)
                for dst, src in zip(self.bufs[nxt_buf], source(order[s + 1])):
                    # The receive buffers are the emulator's own; a source of
                    # their shape and dtype, contiguous on the GPU, needs no
                    # further Python checks (the library checks the rest).
                    if (isinstance(src, torch.Tensor) and src.shape == dst.shape and
                            src.dtype == dst.dtype and src.is_cuda and src.is_contiguous()):
                        _lib.stage_block_checked(dst, src, copy, alone=alone)
                    else:
                        _lib.stage_block(dst, src, copy, alone=alone)
                self.ev_ready[nxt_buf].record(copy)
            if cur_buf is not None:
                self.ev_ready[cur_buf].wait(comp)
            self.last_stop = None
            fold(s, j, cur)
            if cur_buf is not None:
                # The buffer is free once the visit's last kernel has ended: a
                # timed fold's stop event (bound to that kernel's dispatch)
                # says so without another marker on the compute stream.
                if self.last_stop is not None:
                    self.last_stop.wait(copy)
                else:
                    self.ev_free[cur_buf].record(comp)
                    self.ev_free[cur_buf].wait(copy)
                if drain is not None:
                    drain(j, cur, copy)
                if self.free_hook is not None:
                    self.free_hook(cur, copy)
            if nxt_buf is not None:
                # The buffer just computed on becomes the next receive target;
                # the copy stream has waited for its free event before refilling it.
                free_buf = cur_buf if cur_buf is not None else 1 - nxt_buf
                cur, cur_buf = self.bufs[nxt_buf], nxt_buf
        if drain is not None:
            self.ev_start.record(copy)
            self.ev_start.wait(comp)

    def _visit_fused(self, order, source, fold, drain, busy) -> None:
        """visit() with the staging carried by the step launches: the copies
        of order[s+1] into the free buffer are handed to the launches of step
        s (see step), all on the compute stream; the stream orders each copy
        after the reads of the buffer it refills and before the step that
        reads it.  Copies no launch took (a skipped block) run alone after the
        step's launches."""
        if drain is not None:
            raise ValueError("fused staging carries no drain: a backward ring stages on the side stream")
        comp = self.compute
        cur = source(order[0])
        cur_buf = None
        free_buf = 0
        for s, j in enumerate(order):
            nxt_buf = None
            self.pending = []
            if s + 1 < len(order):
                nxt_buf = free_buf
                self.pending = list(zip(self.bufs[nxt_buf], source(order[s + 1])))
            self.last_stop = None
            fold(s, j, cur)
            for dst, src in self.pending:
                if (isinstance(src, torch.Tensor) and src.shape == dst.shape and
                        src.dtype == dst.dtype and src.is_cuda and src.is_contiguous()):
                    _lib.stage_block_checked(dst, src, comp, alone=True)
                else:
                    _lib.stage_block(dst, src, comp, alone=True)
            self.pending = []
            if cur_buf is not None and self.free_hook is not None:
                self.free_hook(cur, comp)
            if nxt_buf is not None:
                free_buf = cur_buf if cur_buf is not None else 1 - nxt_buf
                cur, cur_buf = self.bufs[nxt_buf], nxt_buf

    def _take_copies(self, case) -> list:
        """The copies a launched step carries (fused staging): up to
        copies_per_launch of the pending ones."""
        if self.staging != "fused" or case == _lib.RA_CASE_SKIP or not self.pending:
            return []
        take = self.pending[:self.copies_per_launch]
        self.pending = self.pending[self.copies_per_launch:]
        for dst, src in take:
            if not (isinstance(src, torch.Tensor) and src.shape == dst.shape and src.dtype == dst.dtype
                    and src.is_cuda and src.is_contiguous()):
                _lib.check_copies([(dst, src)])
        return take

    def timer_pair(self, case, step_timers, timer_events):
        """(start, stop) timing events for a launch that step_timers records,
        or (None, None).  The stop event also marks the end of the visit's
        compute for the staging protocol (visit)."""
        if step_timers is None or case == _lib.RA_CASE_SKIP:
            return None, None
        if timer_events is not None:
            e0, e1 = next(timer_events), next(timer_events)
        else:
            e0, e1 = Event(timing=True), Event(timing=True)
        step_timers.append((case, e0, e1))
        self.last_stop = e1
        return e0, e1

    def step(self, st, q, k, v, i, j, num_blocks, causal, scale, case, step_timers=None,
             timer_events=None, flags=0, out=(None, None), checked=False, strided=False) -> None:
        """One ra_step (ra_step_ex with flags) on the compute stream; with
        step_timers (see run), ra_step_timed binds a pair of timing events to
        the step kernel's dispatch.  checked: the operands passed
        _lib.check_step already (see run).  strided: q, k, v, the state and
        the outputs may be row ranges of longer blocks (ra_step_strided)."""
        e0, e1 = self.timer_pair(case, step_timers, timer_events)
        copies = self._take_copies(case)
        if strided:
            _lib.step_strided(st, q, k, v, i, j, num_blocks, causal, scale, copies, self.compute,
                              flags=flags, o_out=out[0], lse_out=out[1], start=e0, stop=e1)
            return
        if copies:
            launch = _lib.step_staged_checked if checked else _lib.step_staged
            launch(st, q, k, v, i, j, num_blocks, causal, scale, copies, self.compute, flags=flags,
                   o_out=out[0], lse_out=out[1], start=e0, stop=e1)
            return
        launch = _lib.step_checked if checked else _lib.step
        launch(st, q, k, v, i, j, num_blocks, causal, scale, self.compute, flags=flags,
               o_out=out[0], lse_out=out[1], start=e0, stop=e1)

    def run(self, st: _lib.State, q: torch.Tensor, kv_source: Callable[[int], tuple],
            rank: int, num_blocks: int, causal: bool, scale: float,
            order: Sequence[int] | None = None, init: bool = True,
            step_timers: list | None = None, timer_events=None, finalize_out=None,
            key_split: int = 1) -> list:
        """Contiguous partition: fold the blocks of `order` (default: the ring
        order of `rank`) into st.

        kv_source(j) returns the resident (K_j, V_j) device tensors.
        step_timers, if given, receives (case, start_event, end_event) per
        launched step, recorded on the compute stream around the launch;
        timer_events, if given, is an iterator of timing events created
        beforehand (two per launched step), so that no event is created while
        work is being enqueued.
        finalize_out = (o_out, lse_out), if given, fuses the ring's init and
        finalize into its first and last launched steps (ra_step_ex): the
        first starts from the empty state (when init), the last writes
        o_out, lse_out as finalize would, instead of the state.
        key_split > 1 (no causal mask; query batch 1): kv_source(j) returns
        the blocks in split_keys layout [key_split, H, c / key_split, d], st
        has batch key_split (one partial state per key range), every step
        reads the one query block for all of them (RA_STEP_Q_BROADCAST), and
        finalize_out, if given, is written by one ra_merge_finalize over the
        key_split partial states after the last step.
        Returns the causal case of each step.
        """
        if key_split > 1 and (causal or q.shape[0] != 1 or st.shape[0] != key_split):
            raise ValueError("key_split needs no causal mask, a query batch of 1 and a state batch of key_split")
        order = ring_order(rank, num_blocks) if order is None else list(order)
        all_cases = [_lib.step_case(rank, j, num_blocks, causal) for j in order]
        launched = [s for s, c in enumerate(all_cases) if c != _lib.RA_CASE_SKIP]
        fuse = finalize_out is not None and len(launched) > 0
        fuse_finalize = fuse and key_split == 1
        if init and not fuse:
            _lib.state_init(st, self.compute)
        cases = []
        # Every step passes the state, the query block, the finalize outputs
        # and either the ring's first block (used where it lies) or one of the
        # receive buffers (every later block is staged into them): checked
        # once here, so the steps go to the library without Python checks.
        all_flags = ((_lib.RA_STEP_Q_BROADCAST if key_split > 1 else 0) |
                     (_lib.RA_STEP_FINALIZE if fuse_finalize else 0))
        fin = finalize_out if fuse_finalize else (None, None)
        first = kv_source(order[0])
        _lib.check_step(st, q, first[0], first[1], all_flags, *fin)
        if len(order) > 1:
            _lib.check_step(st, q, self.bufs[0][0], self.bufs[0][1], all_flags, *fin)

        def fold(s, j, kv):
            case = all_cases[s]
            flags = _lib.RA_STEP_Q_BROADCAST if key_split > 1 else 0
            if fuse and init and s == launched[0]:
                flags |= _lib.RA_STEP_FRESH
            if fuse_finalize and s == launched[-1]:
                flags |= _lib.RA_STEP_FINALIZE
            self.step(st, q, kv[0], kv[1], rank, j, num_blocks, causal, scale, case,
                      step_timers, timer_events, flags,
                      finalize_out if flags & _lib.RA_STEP_FINALIZE else (None, None), checked=True)
            cases.append(case)

        self.visit(order, kv_source, fold, busy=lambda s: all_cases[s] != _lib.RA_CASE_SKIP)
        if finalize_out is not None:
            if key_split > 1:
                _lib.merge_finalize(st, key_split, stream=self.compute, o_out=finalize_out[0],
                                    lse_out=finalize_out[1])
            elif not fuse:
                _lib.finalize(st, stream=self.compute, o_out=finalize_out[0], lse_out=finalize_out[1])
        return cases


    def run_backward(self, q, dout, lse, delta, dq, source: Callable[[int], tuple],
                     rank: int, num_blocks: int, causal: bool, scale: float,
                     step_timers: list | None = None, timer_events=None) -> list:
        """Backward ring of `rank` ("Ring Attention：...", section "Backward
        需要让梯度也沿环传播"): dq (fp32, zeroed by the caller) accumulates the
        contributions of every visiting block; source(j) returns block j's
        resident (K_j, V_j, dK_j, dV_j), of which the fp32 dK_j, dV_j travel
        with the block: they are staged in with K_j, V_j, the step adds this
        rank's contribution, and they are sent on (copied back to the resident
        tensors) after the step.  Needs extra_specs for dK, dV at construction.
        Returns the causal case of each step."""
        order = ring_order(rank, num_blocks)
        cases = []

        def fold(s, j, t):
            case = _lib.step_case(rank, j, num_blocks, causal)
            e0, e1 = self.timer_pair(case, step_timers, timer_events)
            _lib.bwd_step(q, dout, lse, delta, t[0], t[1], dq, t[2], t[3], rank, j, num_blocks,
                          causal, scale, self.compute, start=e0, stop=e1)
            cases.append(case)

        def drain(j, t, stream):
            dk, dv = source(j)[2:4]
            _lib.stage_block(dk, t[2], stream)
            _lib.stage_block(dv, t[3], stream)

        self.visit(order, source, fold, drain,
                   busy=lambda s: _lib.step_case(rank, order[s], num_blocks, causal) != _lib.RA_CASE_SKIP)
        return cases


def zigzag_launches(rank: int, ranks: int, causal: bool) -> list:
    """Per ring step: (visiting rank j, [(q_lo, q_n, kv_lo, kv_n, case)]), the
    launches of ZigzagRing.run_block.  A rank's block holds its two sub-blocks
    in position order (sub-block 0 the earlier), so do the visiting ones; a
    launch folds query sub-blocks [q_lo, q_lo + q_n) against key/value
    sub-blocks [kv_lo, kv_lo + kv_n) with case RA_CASE_FULL (no mask) or
    RA_CASE_DIAG (the causal mask of the joined block, which is the mask of
    its positions because they increase along it).  Under the causal mask a
    visit of the rank's own block is one diagonal launch, of an earlier rank
    one launch of both query sub-blocks against the earlier visiting
    sub-block, of a later rank one launch of the later query sub-block
    against both (zigzag_plan's pair cases, joined); pairs that join into
    no such rectangle stay one launch each."""
    F, D, S = _lib.RA_CASE_FULL, _lib.RA_CASE_DIAG, _lib.RA_CASE_SKIP
    out = []
    for j, prods in zigzag_plan(rank, ranks, causal):
        c = {(a, b): case for a, b, case in prods}
        if all(v == F for v in c.values()):
            launches = [(0, 2, 0, 2, F)]
        elif c == {(0, 0): D, (0, 1): S, (1, 0): F, (1, 1): D}:
            launches = [(0, 2, 0, 2, D)]
        elif c[0, 0] == c[0, 1] == S and c[1, 0] == c[1, 1] == F:
            launches = [(1, 1, 0, 2, F)]
        elif c[0, 1] == c[1, 1] == S and c[0, 0] == c[1, 0] == F:
            launches = [(0, 2, 0, 1, F)]
        else:
            launches = [(a, 1, b, 1, case) for a, b, case in prods if case != S]
        out.append((j, launches))
    return out


def launch_pairs(launch, sub_rows: int) -> int:
    """(query, key) pairs one zigzag_launches launch folds per (batch, head)
    entry, for sub-blocks of sub_rows rows."""
    q_lo, q_n, kv_lo, kv_n, case = launch[:5]
    if case == _lib.RA_CASE_DIAG:
        r = q_n * sub_rows
        return r * (r + 1) // 2
    if case == _lib.RA_CASE_FULL:
        return q_n * kv_n * sub_rows * sub_rows
    return 0


def _split_rows(launch) -> list:
    """A launch of both query sub-blocks as launches of one each (the pairs of
    the joined launch, each row sub-block's FULL pairs joined again)."""
    q_lo, q_n, kv_lo, kv_n, case = launch
    if q_n == 1:
        return [launch]
    if case == _lib.RA_CASE_FULL:
        return [(0, 1, kv_lo, kv_n, case), (1, 1, kv_lo, kv_n, case)]
    # the joined diagonal: (0, 0) diagonal, (1, 0) full, (1, 1) diagonal
    return [(0, 1, 0, 1, case), (1, 1, 0, 1, _lib.RA_CASE_FULL), (1, 1, 1, 1, case)]


def zigzag_fused_launches(rank: int, ranks: int, causal: bool) -> list:
    """zigzag_launches with each query sub-block's first and last launch
    marked: per step (j, [(q_lo, q_n, kv_lo, kv_n, case, fresh, final)]).  A
    launch of both sub-blocks that is the first (last) for one of them only
    is split per sub-block, so that RA_STEP_FRESH (RA_STEP_FINALIZE) applies
    to exactly the rows it should."""
    steps = [(j, list(ls)) for j, ls in zigzag_launches(rank, ranks, causal)]

    def where(pick_last):
        found = {}
        order = [(s, n) for s, (_, ls) in enumerate(steps) for n in range(len(ls))]
        for s, n in (reversed(order) if pick_last else order):
            q_lo, q_n = steps[s][1][n][:2]
            for p in range(q_lo, q_lo + q_n):
                found.setdefault(p, (s, n))
        return found

    while True:
        first, last = where(False), where(True)
        split = False
        for s, (_, ls) in enumerate(steps):
            for n in reversed(range(len(ls))):
                q_lo, q_n = ls[n][:2]
                for found in (first, last):
                    marks = [found.get(p) == (s, n) for p in range(q_lo, q_lo + q_n)]
                    if any(marks) and not all(marks):
                        ls[n:n + 1] = _split_rows(ls[n])
                        split = True
                        break
        if not split:
            break
    out = []
    for s, (j, ls) in enumerate(steps):
        out.append((j, [(*l, first.get(l[0]) == (s, n), last.get(l[0]) == (s, n))
                        for n, l in enumerate(ls)]))
    return out


class ZigzagRing:
    """One rank's ring under the zigzag partition.

    sub_shape: [batch, heads, rows, head_dim] of one sub-block (rows = c / 2
    for c tokens per rank).  The rank's query and state are two sub-block
    tensors each (sub-blocks zigzag_blocks(rank, P)); kv_source(j) returns
    (K_a, K_b, V_a, V_b) of rank j's two sub-blocks zigzag_blocks(j, P).
    """

    def __init__(self, sub_shape, dtype, device="cuda", compute_stream=None, copy_stream=None,
                 backward: bool = False, staging: str = "side"):
        # backward: also stage the fp32 dK, dV of the visiting rank's two sub-blocks.
        # staging: as for RingEmulator ("fused": forward rings only).
        extra = [(tuple(sub_shape), torch.float32)] * 4 if backward else ()
        self.emu = RingEmulator(sub_shape, dtype, device, compute_stream, copy_stream,
                                tensors_per_visit=4, extra_specs=extra, staging=staging)
        self.backward = backward

    @property
    def compute(self):
        return self.emu.compute

    def run(self, states: Sequence[_lib.State], qs: Sequence[torch.Tensor],
            kv_source: Callable[[int], tuple], rank: int, ranks: int, causal: bool,
            scale: float, init: bool = True, step_timers: list | None = None,
            timer_events=None, finalize_outs=None) -> list:
        """Fold every visiting rank's two sub-blocks into the two states.
        finalize_outs = [(o_out, lse_out)] * 2, if given, fuses each state's
        init and finalize into its first and last launched piece product, as
        RingEmulator.run does.  Returns zigzag_plan(rank, ranks, causal)."""
        plan = zigzag_plan(rank, ranks, causal)
        mine = zigzag_blocks(rank, ranks)
        prods = [(s, a, b) for s, (_, ps) in enumerate(plan) for a, b, c in ps
                 if c != _lib.RA_CASE_SKIP]
        firsts = {a: next((p for p in prods if p[1] == a), None) for a in range(2)}
        lasts = {a: next((p for p in reversed(prods) if p[1] == a), None) for a in range(2)}
        fuse = [finalize_outs is not None and firsts[a] is not None for a in range(2)]
        for a, st in enumerate(states):
            if init and not fuse[a]:
                _lib.state_init(st, self.compute)

        def fold(s, j, kv):
            theirs = zigzag_blocks(j, ranks)
            for a, b, case in plan[s][1]:
                flags = 0
                if fuse[a] and init and (s, a, b) == firsts[a]:
                    flags |= _lib.RA_STEP_FRESH
                if fuse[a] and (s, a, b) == lasts[a]:
                    flags |= _lib.RA_STEP_FINALIZE
                self.emu.step(states[a], qs[a], kv[b], kv[2 + b], mine[a], theirs[b],
                              2 * ranks, causal, scale, case, step_timers, timer_events, flags,
                              finalize_outs[a] if flags else (None, None))

        self.emu.visit([j for j, _ in plan], kv_source, fold,
                       busy=lambda s: any(c != _lib.RA_CASE_SKIP for _, _, c in plan[s][1]))
        if finalize_outs is not None:
            for a, st in enumerate(states):
                if not fuse[a]:
                    _lib.finalize(st, stream=self.compute, o_out=finalize_outs[a][0],
                                  lse_out=finalize_outs[a][1])
        return plan

    def run_block(self, st: _lib.State, q: torch.Tensor, kv_source: Callable[[int], tuple],
                  rank: int, ranks: int, causal: bool, scale: float, init: bool = True,
                  step_timers: list | None = None, timer_events=None, finalize_out=None) -> list:
        """The forward ring on whole blocks: q [batch, heads, 2*sub_rows,
        head_dim] holds the rank's sub-blocks zigzag_blocks(rank, ranks) in
        position order within each (batch, head) entry, st is its state
        (2*sub_rows rows), kv_source(j) returns (K_j, V_j) of rank j in the
        same layout.  Each visit is the launches of zigzag_launches, row ranges
        of these blocks (ra_step_strided): one per visit under the causal mask
        where run() needs two to four.  finalize_out = (o_out, lse_out) of the
        whole block, if given, fuses the state's init and finalize into each
        sub-block's first and last launch.  Returns the launches per step."""
        emu = self._block_emulator(tuple(q.shape), q.dtype, q.device)
        if q.shape[2] % 2:
            raise ValueError(f"a block of two equal sub-blocks has an even row count, got {q.shape[2]}")
        half = q.shape[2] // 2
        plan = zigzag_fused_launches(rank, ranks, causal)
        # Fusing needs a first and a last launch for each sub-block.
        fuse = finalize_out is not None and all(
            any(l[0] <= p < l[0] + l[1] for _, ls in plan for l in ls) for p in range(2))
        if init and not fuse:
            _lib.state_init(st, emu.compute)

        def rows(t, lo, n):
            return t[:, :, lo * half:(lo + n) * half]

        def fold(s, j, kv):
            for q_lo, q_n, kv_lo, kv_n, case, first, last in plan[s][1]:
                flags = 0
                if fuse and init and first:
                    flags |= _lib.RA_STEP_FRESH
                if fuse and last:
                    flags |= _lib.RA_STEP_FINALIZE
                out = ((rows(finalize_out[0], q_lo, q_n), rows(finalize_out[1], q_lo, q_n))
                       if flags & _lib.RA_STEP_FINALIZE else (None, None))
                diag = case == _lib.RA_CASE_DIAG
                emu.step(st.row_slice(q_lo * half, q_n * half), rows(q, q_lo, q_n),
                         rows(kv[0], kv_lo, kv_n), rows(kv[1], kv_lo, kv_n), 0, 0, 1, diag, scale,
                         case, step_timers, timer_events, flags, out, strided=True)

        emu.visit([j for j, _ in plan], kv_source, fold, busy=lambda s: bool(plan[s][1]))
        if finalize_out is not None and not fuse:
            _lib.finalize(st, stream=emu.compute, o_out=finalize_out[0], lse_out=finalize_out[1])
        return plan

    def _block_emulator(self, shape, dtype, device) -> RingEmulator:
        """The two-tensor (K, V of whole blocks) emulator of run_block, on the
        same streams as the sub-block one, built on first use."""
        em = getattr(self, "_blk", None)
        if em is None or em.shape != shape or em.dtype != dtype:
            em = RingEmulator(shape, dtype, device, self.emu.compute, self.emu.copy,
                              staging=self.emu.staging)
            self._blk = em
        return em

    def run_backward(self, qs: Sequence[torch.Tensor], douts: Sequence[torch.Tensor],
                     lses: Sequence[torch.Tensor], deltas: Sequence[torch.Tensor],
                     dqs: Sequence[torch.Tensor], source: Callable[[int], tuple], rank: int,
                     ranks: int, causal: bool, scale: float, step_timers: list | None = None,
                     timer_events=None) -> list:
        """Backward ring of `rank` under the zigzag partition: the two fp32 dq
        sub-block tensors (zeroed by the caller) accumulate every visiting
        sub-block's contribution; source(j) returns (K_a, K_b, V_a, V_b, dK_a,
        dK_b, dV_a, dV_b) of rank j's sub-blocks zigzag_blocks(j, ranks), whose
        fp32 dK, dV travel with them (staged in, updated by this rank's piece
        products, sent on).  Needs backward=True at construction.  Returns
        zigzag_plan(rank, ranks, causal)."""
        if not self.backward:
            raise RuntimeError("ZigzagRing.run_backward needs backward=True at construction")
        plan = zigzag_plan(rank, ranks, causal)
        mine = zigzag_blocks(rank, ranks)
        comp = self.compute

        def fold(s, j, t):
            theirs = zigzag_blocks(j, ranks)
            for a, b, case in plan[s][1]:
                e0, e1 = self.emu.timer_pair(case, step_timers, timer_events)
                _lib.bwd_step(qs[a], douts[a], lses[a], deltas[a], t[b], t[2 + b], dqs[a],
                              t[4 + b], t[6 + b], mine[a], theirs[b], 2 * ranks, causal, scale, comp,
                              start=e0, stop=e1)

        def drain(j, t, stream):
            for dst, src in zip(source(j)[4:8], t[4:8]):
                _lib.stage_block(dst, src, stream)

        self.emu.visit([j for j, _ in plan], source, fold, drain,
                       busy=lambda s: any(c != _lib.RA_CASE_SKIP for _, _, c in plan[s][1]))
        return plan
