"""Independent fp64 model of the blockwise online-softmax recurrence.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  It exists to pin the dense
oracle: folding blocks in any order, merging two partial states and skipping
fully masked blocks must all land on the dense answer.  It is written from the
pages' description of the per-query running state, not from any kernel.

Sources (page title, then section):
  * "Ring Attention Math Deep", section "The online-softmax identity that makes
    streaming legal": per query keep a running maximum m, a denominator l of
    exp(s - m) and an unnormalised output o of exp(s - m) v; a new block raises
    m to m' and rescales the old l and o by exp(m - m') before adding its own
    terms; after the last block the output is o / l.
  * "Ring Attention Paper Breakdown: Blockwise Distributed Transformers for
    Near-Infinite Context", section 3 "Cross-Device Online Softmax Accumulator
    Math": the same seven-step update written per block (row max, new running
    max, rescale factor, block exponentials, normaliser, output).
  * aicassindra architecture article, section "The architecture: every piece
    explained": two partial results merge by taking the larger maximum and
    rescaling each side by exp(its max - new max) before adding; the empty
    state (m=-inf, l=0, o=0) is the identity of that merge (section "End-to-end
    flow").

Reading taken where the pages are silent: when the old maximum is -inf the
rescale factor is 0 (the worked example prints alpha = 0 for the first block);
a block that contributes no allowed key leaves the state unchanged, so
exp(-inf - (-inf)) is never formed.
"""
from __future__ import annotations

import numpy as np

__all__ = ["State", "empty_state", "fold_block", "merge", "finalize"]


class State:
    """Running (m, l, o) for R query rows: m [R], l [R], o [R, dv] in float64."""

    def __init__(self, m, l, o):
        self.m = m
        self.l = l
        self.o = o

    def copy(self):
        return State(self.m.copy(), self.l.copy(), self.o.copy())


def empty_state(rows: int, dv: int) -> State:
    return State(np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, dv)))


def fold_block(st: State, s_block, v_block, allowed=None, trace=None) -> State:
    """Fold one visiting block into the state.

    s_block [R, n]   already-scaled scores of the R queries against the block
    v_block [n, dv]  the block's values
    allowed [R, n]   optional boolean mask (causal); disallowed terms are absent
    trace            optional list; receives a dict of this fold's intermediates
    """
    s = np.asarray(s_block, dtype=np.float64)
    v = np.asarray(v_block, dtype=np.float64)
    if allowed is None:
        allowed = np.ones(s.shape, dtype=bool)
    m_new = st.m.copy()
    l_new = st.l.copy()
    o_new = st.o.copy()
    alphas = np.ones(len(st.m))
    for r in range(s.shape[0]):
        sel = allowed[r]
        if not sel.any():
            continue                                  # block absent for this row
        srow = s[r, sel]
        m_prev = st.m[r]
        m_cur = max(m_prev, float(srow.max()))
        alpha = 0.0 if m_prev == -np.inf else float(np.exp(m_prev - m_cur))
        p = np.exp(srow - m_cur)
        m_new[r] = m_cur
        l_new[r] = alpha * st.l[r] + p.sum()
        o_new[r] = alpha * st.o[r] + p @ v[sel]
        alphas[r] = alpha
    if trace is not None:
        trace.append({"m": m_new.copy(), "alpha": alphas, "l": l_new.copy(),
                      "o": o_new.copy()})
    return State(m_new, l_new, o_new)


def merge(a: State, b: State) -> State:
    """Merge two partial states over disjoint key sets."""
    m = np.maximum(a.m, b.m)
    l = np.zeros_like(a.l)
    o = np.zeros_like(a.o)
    for r in range(len(m)):
        if m[r] == -np.inf:
            continue                                  # both sides empty
        wa = 0.0 if a.m[r] == -np.inf else float(np.exp(a.m[r] - m[r]))
        wb = 0.0 if b.m[r] == -np.inf else float(np.exp(b.m[r] - m[r]))
        l[r] = wa * a.l[r] + wb * b.l[r]
        o[r] = wa * a.o[r] + wb * b.o[r]
    return State(m, l, o)


def finalize(st: State):
    """Return (o / l, m + ln l); empty rows give (0, -inf)."""
    out = np.zeros_like(st.o)
    lse = np.full(len(st.m), -np.inf)
    nz = st.l > 0
    out[nz] = st.o[nz] / st.l[nz, None]
    lse[nz] = st.m[nz] + np.log(st.l[nz])
    return out, lse
