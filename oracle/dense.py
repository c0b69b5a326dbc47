"""Dense fp64 softmax attention: the plain definition the ring computes.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Sources (page title, then section):
  * "Ring Attention Math Deep" (Belgavi.AI Lab), section "Why one device runs
    out of room": the scores are Q K^T / sqrt(d_k) over the whole sequence.
  * same page, section "The online-softmax identity that makes streaming
    legal": the output is a ratio of exp-weighted sums in which any common
    constant cancels; the row maximum is only a choice for numerical safety.
  * "Ring Attention：把超长序列沿设备环流动", section "Causal Attention
    让环不再完全对称": a query at global position p may use keys at global
    positions <= p.  The inclusive boundary matches the end-to-end flow of the
    aicassindra architecture article (local query p uses local keys 0..p) and
    the causal section of "RingAttention: Scaling LLM Context to 10M Tokens".
  * "Ring Attention：把超长序列沿设备环流动", section "Backward
    需要让梯度也沿环传播": a per-row log-sum-exp is what the backward keeps.
    It is read here as the natural log of the sum of exp(scaled score) over
    the allowed keys.

A row with no allowed key (only possible for partial key sets) gets O = 0 and
LSE = -inf: the pages are silent; this is the value of an empty sum.

No online recurrence, blocking or reordering happens here: per row chunk the
whole allowed score row is formed with one matrix product, masked, shifted,
exponentiated, summed and multiplied into V.
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_bits_to_f64", "attention", "ring_positions"]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64.

    bfloat16 is the upper half of an IEEE binary32, so widening is exact.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.view(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def ring_positions(block: int, rows: int) -> np.ndarray:
    """Global token positions of contiguous block `block` of length `rows`.

    Contiguous sharding: block i owns tokens [i*rows, (i+1)*rows)
    ("Ring Attention Math Deep", section "Sharding the sequence: what each
    device holds").
    """
    return np.arange(block * rows, (block + 1) * rows, dtype=np.int64)


def attention(q, k, v, q_pos, k_pos, causal: bool, scale: float,
              shift="max", row_chunk: int = 64):
    """Dense masked softmax attention in float64.

    q      [H, R, d]   queries (any real dtype; converted to float64)
    k      [H, N, d]   keys
    v      [H, N, dv]  values
    q_pos  [R]         global positions of the query rows
    k_pos  [N]         global positions of the keys
    causal             if true, key n is allowed for query r iff k_pos[n] <= q_pos[r]
    scale              multiplies q.k (1/sqrt(d) in the pages)
    shift              "max" (the row maximum over allowed keys) or a float
                       constant subtracted before exponentiation; the result
                       does not depend on it (softmax shift invariance)

    Returns (O [H, R, dv], LSE [H, R]) in float64, LSE = natural log of the
    sum of exp(scaled score) over allowed keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    H, R, d = q.shape
    N = k.shape[1]
    dv = v.shape[2]
    assert k.shape == (H, N, d) and v.shape[:2] == (H, N)
    assert q_pos.shape == (R,) and k_pos.shape == (N,)

    out = np.zeros((H, R, dv), dtype=np.float64)
    lse = np.full((H, R), -np.inf, dtype=np.float64)
    if R == 0 or N == 0:
        return out, lse

    for h in range(H):
        for r0 in range(0, R, row_chunk):
            r1 = min(R, r0 + row_chunk)
            s = (q[h, r0:r1] @ k[h].T) * scale            # [rc, N] scaled scores
            if causal:
                allowed = k_pos[None, :] <= q_pos[r0:r1, None]
            else:
                allowed = np.ones(s.shape, dtype=bool)
            s = np.where(allowed, s, -np.inf)
            any_allowed = allowed.any(axis=1)
            if isinstance(shift, str):
                assert shift == "max"
                c = np.max(s, axis=1)                      # -inf for empty rows
                c = np.where(any_allowed, c, 0.0)
            else:
                c = np.full(r1 - r0, float(shift))
            w = np.exp(s - c[:, None])                     # masked -> exp(-inf) = 0
            l = w.sum(axis=1)
            num = w @ v[h]
            with np.errstate(divide="ignore", invalid="ignore"):
                o = num / l[:, None]
                row_lse = c + np.log(l)
            o[~any_allowed] = 0.0
            row_lse[~any_allowed] = -np.inf
            out[h, r0:r1] = o
            lse[h, r0:r1] = row_lse
    return out, lse
