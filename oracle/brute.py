"""50-digit decimal brute force of softmax attention for tiny inputs.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Straight from the definition in "RingAttention: Scaling LLM Context to 10M
Tokens", section "Incremental Online Softmax Accumulation" (O = softmax(Q K^T /
sqrt(d)) V) with the causal rule of its section "Causal Masking: Striped and
Zig-Zag RingAttention" (token t sees keys j <= t).  No maximum is subtracted:
with 50 significant digits and tiny scores nothing overflows, so this checks
the shifted fp64 oracle against the unshifted formula.
"""
from __future__ import annotations

from decimal import Decimal, getcontext

__all__ = ["attention_decimal"]


def attention_decimal(q, k, v, q_pos, k_pos, causal, scale, digits=50):
    """q [R][d], k [N][d], v [N][dv] as nested lists of floats (one head).

    Returns (O [R][dv], LSE [R]) as Decimals; rows with no allowed key give
    O = 0 and LSE = None.
    """
    getcontext().prec = digits
    sc = Decimal(scale)
    out, lse = [], []
    for r, qr in enumerate(q):
        num = [Decimal(0)] * len(v[0])
        den = Decimal(0)
        for n, kn in enumerate(k):
            if causal and k_pos[n] > q_pos[r]:
                continue
            s = sum(Decimal(a) * Decimal(b) for a, b in zip(qr, kn)) * sc
            w = s.exp()
            den += w
            num = [acc + w * Decimal(x) for acc, x in zip(num, v[n])]
        if den == 0:
            out.append([Decimal(0)] * len(v[0]))
            lse.append(None)
        else:
            out.append([x / den for x in num])
            lse.append(den.ln())
    return out, lse
