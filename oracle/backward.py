"""Dense fp64 backward of softmax attention, and the per-block contribution the
ring backward accumulates.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Sources (page title, then section):
  * "Ring Attention：把超长序列沿设备环流动", section "Backward
    需要让梯度也沿环传播": every (query block, key/value block) interaction
    contributes to the gradients; the query owner accumulates dQ locally, the
    dK and dV of a key/value block accumulate while it travels the ring and
    return to its owner; like the FlashAttention backward, the per-row
    log-sum-exp saved by the forward lets each block recompute its scores and
    probabilities instead of storing the attention matrix.
  * The forward it differentiates is the one of dense.py (scores scale*q.k,
    inclusive causal mask, softmax over the allowed keys, P V).

The pages give no gradient formulas; these are the chain rule applied to that
forward (the plain definition), for a loss L with dL/dO = dO:
    P = softmax(S) over allowed keys,  O = P V
    dV = P^T dO
    dP = dO V^T
    D_i = sum_k P_ik dP_ik = dO_i . O_i
    dS = P * (dP - D)            (elementwise; dS = 0 where masked)
    dQ = scale * dS K,   dK = scale * dS^T Q
A row with no allowed key has P = 0 and contributes nothing.

block_backward is the same formula restricted to one key block, with P
recomputed as exp(S - LSE) from the saved per-row LSE and D taken as given:
the step a ring rank performs.  Summing it over key blocks must give the dense
result; that is one of the pins in tests/test_oracle_backward.py.
"""
from __future__ import annotations

import numpy as np

from .dense import attention

__all__ = ["attention_backward", "block_backward", "row_dot", "forward_for_backward"]


def _mask(q_pos, k_pos, causal):
    qp = np.asarray(q_pos, dtype=np.int64)
    kp = np.asarray(k_pos, dtype=np.int64)
    if causal:
        return kp[None, :] <= qp[:, None]
    return np.ones((len(qp), len(kp)), dtype=bool)


def attention_backward(q, k, v, do, q_pos, k_pos, causal: bool, scale: float):
    """Gradients of dense attention.  q, do [H, R, d]; k, v [H, N, d].

    Returns dq [H, R, d], dk [H, N, d], dv [H, N, d] in float64.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    allowed = _mask(q_pos, k_pos, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(q.shape[0]):
        s = scale * (q[h] @ k[h].T)
        s = np.where(allowed, s, -np.inf)
        has = allowed.any(axis=1)
        m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
        w = np.where(allowed, np.exp(s - m[:, None]), 0.0)
        den = w.sum(axis=1)
        p = np.divide(w, den[:, None], out=np.zeros_like(w), where=den[:, None] > 0)
        o = p @ v[h]
        dv[h] = p.T @ do[h]
        dp = do[h] @ v[h].T
        d_row = np.sum(do[h] * o, axis=1)
        ds = p * (dp - d_row[:, None])
        dq[h] = scale * (ds @ k[h])
        dk[h] = scale * (ds.T @ q[h])
    return dq, dk, dv


def row_dot(do, o):
    """D = rowsum(dO * O) [H, R]: the per-row term of dS, from the forward output."""
    return np.sum(np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64), axis=-1)


def block_backward(q, k, v, do, lse, d_row, q_pos, k_pos, causal: bool, scale: float):
    """Contribution of one key/value block to (dQ, dK, dV), with the probabilities
    recomputed from the saved LSE [H, R] and D [H, R] given.

    Returns dq [H, R, d] (this block's part of the query gradient) and dk, dv
    [H, N, d] (this query block's part of the key/value gradients).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    lse = np.asarray(lse, dtype=np.float64)
    d_row = np.asarray(d_row, dtype=np.float64)
    allowed = _mask(q_pos, k_pos, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(q.shape[0]):
        s = scale * (q[h] @ k[h].T)
        finite = np.isfinite(lse[h])[:, None] & allowed
        p = np.where(finite, np.exp(np.where(finite, s - lse[h][:, None], 0.0)), 0.0)
        dv[h] = p.T @ do[h]
        dp = do[h] @ v[h].T
        ds = p * (dp - d_row[h][:, None])
        dq[h] = scale * (ds @ k[h])
        dk[h] = scale * (ds.T @ q[h])
    return dq, dk, dv


def forward_for_backward(q, k, v, q_pos, k_pos, causal: bool, scale: float):
    """The forward output and LSE the backward needs (dense.attention)."""
    return attention(q, k, v, q_pos, k_pos, causal, scale)
