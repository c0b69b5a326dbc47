"""Pins of the CPU fp64 oracle against what the pages and mathematics fix.

Each pin is written as a function of an `attention` implementation so that the
last test can plant plausible mistakes in a copy of the oracle's source (on the
CPU) and show that every such mutant fails at least one pin.
"""
import itertools
import json
import math
import os
import re

import numpy as np
import pytest

from oracle import blockwise, brute, dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _worked():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand_case(seed, H, P, c, d, dv=None):
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    q = rng.standard_normal((H, c, d))
    ks = [rng.standard_normal((H, c, d)) for _ in range(P)]
    vs = [rng.standard_normal((H, c, dv)) for _ in range(P)]
    return q, ks, vs


def _dense_rank(att, q, ks, vs, i, blocks, causal, scale, shift="max"):
    c = q.shape[1]
    k = np.concatenate([ks[j] for j in blocks], axis=1)
    v = np.concatenate([vs[j] for j in blocks], axis=1)
    kp = np.concatenate([dense.ring_positions(j, c) for j in blocks])
    return att(q, k, v, dense.ring_positions(i, c), kp, causal, scale, shift=shift)


# ---------------------------------------------------------------- pins ----------

def pin_worked_example(att):
    """'Ring Attention Math Deep', 'A worked numeric example': out = 2.621."""
    g = _worked()
    s = [x for b in g["blocks"] for x in b["scores"]]
    vals = [x for b in g["blocks"] for x in b["values"]]
    q = np.ones((1, 1, 1))
    k = np.array(s, dtype=np.float64).reshape(1, 4, 1)
    v = np.array(vals, dtype=np.float64).reshape(1, 4, 1)
    o, lse = att(q, k, v, np.array([10]), np.arange(4), False, 1.0)
    half_ulp = 0.5 * 10 ** (-g["printed_decimals"])
    assert abs(o[0, 0, 0] - g["output"]) <= half_ulp
    # LSE is not printed; its value from the 50-digit brute force of the
    # same definition must agree.
    _, lse_dec = brute.attention_decimal([[1.0]], [[x] for x in s], [[x] for x in vals],
                                         [10], [0, 1, 2, 3], False, 1.0)
    assert abs(lse[0, 0] - float(lse_dec[0])) < 1e-12
    assert abs(lse[0, 0] - 3.440190) < 1e-6


def pin_closed_forms(att):
    rng = np.random.default_rng(7)
    H, c, d, P = 2, 5, 3, 3
    q, ks, vs = _rand_case(11, H, P, c, d)
    scale = 0.37
    # causal rank 0 row 0 sees only key 0: O = v_0, LSE = s_00
    o, lse = _dense_rank(att, q, ks, vs, 0, range(P), True, scale)
    for h in range(H):
        assert np.allclose(o[h, 0], vs[0][h, 0], rtol=0, atol=1e-14)
        assert abs(lse[h, 0] - scale * q[h, 0] @ ks[0][h, 0]) < 1e-14
    # rank 0 row r sees keys 0..r of block 0 only; with all keys equal the
    # weights are uniform: O = mean of those values, LSE = s + ln(r+1)
    keq = [np.repeat(ks[j][:, :1], c, axis=1) for j in range(P)]
    o, lse = _dense_rank(att, q, keq, vs, 0, range(P), True, scale)
    for h in range(H):
        for r in range(c):
            assert np.allclose(o[h, r], vs[0][h, :r + 1].mean(axis=0), atol=1e-13)
            s = scale * q[h, r] @ ks[0][h, 0]
            assert abs(lse[h, r] - (s + math.log(r + 1))) < 1e-13
    # all value rows equal u: O = u for every row (non-causal, rank 2)
    u = rng.standard_normal(d)
    vu = [np.broadcast_to(u, (H, c, d)).copy() for _ in range(P)]
    o, _ = _dense_rank(att, q, ks, vu, 2, range(P), False, scale)
    assert np.allclose(o, u, atol=1e-13)
    # every output coordinate lies in the hull of the allowed values
    o, _ = _dense_rank(att, q, ks, vs, 1, range(P), True, scale)
    allowed_v = np.concatenate([vs[0], vs[1]], axis=1)
    assert (o <= allowed_v.max(axis=1, keepdims=True) + 1e-13).all()
    assert (o >= allowed_v.min(axis=1, keepdims=True) - 1e-13).all()


def pin_brute_force(att):
    """Decimal brute force of the unshifted definition, tiny shapes."""
    for P, c, d, causal, seed in itertools.product([1, 2, 4], [1, 2], [1, 4], [False, True], [3]):
        if P * c > 8:
            continue
        q, ks, vs = _rand_case(seed + P * 10 + c, 1, P, c, d, dv=3)
        scale = 1.0 / math.sqrt(d) * 1.3
        for i in range(P):
            o, lse = _dense_rank(att, q, ks, vs, i, range(P), causal, scale)
            k = np.concatenate(ks, axis=1)[0]
            v = np.concatenate(vs, axis=1)[0]
            kp = list(range(P * c))
            qp = list(range(i * c, (i + 1) * c))
            od, ld = brute.attention_decimal(q[0].tolist(), k.tolist(), v.tolist(), qp, kp,
                                             causal, scale)
            for r in range(c):
                for x in range(3):
                    assert abs(o[0, r, x] - float(od[r][x])) <= 1e-13
                assert abs(lse[0, r] - float(ld[r])) <= 1e-13


def pin_torch_sdpa(att):
    """Library cross-check: torch CPU float64 scaled_dot_product_attention."""
    import torch
    import torch.nn.functional as F
    for (H, P, c, d, i, causal) in [(1, 4, 16, 8, 1, True), (3, 3, 9, 5, 2, False),
                                    (2, 4, 7, 6, 3, True)]:
        q, ks, vs = _rand_case(5 + c, H, P, c, d)
        scale = 1.0 / math.sqrt(d)
        o, lse = _dense_rank(att, q, ks, vs, i, range(P), causal, scale)
        tq = torch.from_numpy(q)[None]
        tk = torch.from_numpy(np.concatenate(ks, axis=1))[None]
        tv = torch.from_numpy(np.concatenate(vs, axis=1))[None]
        qp = torch.arange(i * c, (i + 1) * c)
        kp = torch.arange(P * c)
        mask = (kp[None, :] <= qp[:, None]) if causal else torch.ones(c, P * c, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)[0]
        s = (tq @ tk.transpose(-1, -2))[0] * scale
        ref_lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
        assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12)
        assert np.allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-12)


ALL_PINS = [pin_worked_example, pin_closed_forms, pin_brute_force, pin_torch_sdpa]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(dense.attention)


# ------------------------------------------------ recurrence / invariants ------

def test_worked_example_intermediates():
    """Every intermediate the worked example prints, from the blockwise model."""
    g = _worked()
    half = 0.5 * 10 ** (-g["printed_decimals"]) + 1e-12
    st = blockwise.empty_state(1, 1)
    trace = []
    for b, want in zip(g["blocks"], g["after_block"]):
        s = np.array([b["scores"]])
        v = np.array(b["values"])[:, None]
        p = np.exp(s[0] - max(s[0].max(), st.m[0]))
        st = blockwise.fold_block(st, s, v, trace=trace)
        t = trace[-1]
        assert abs(t["m"][0] - want["m"]) <= half
        assert abs(t["alpha"][0] - want["alpha"]) <= half
        assert np.all(np.abs(p - np.array(want["exp"])) <= half)
        assert abs(t["l"][0] - want["l"]) <= half
        assert abs(t["o"][0, 0] - want["o"]) <= half
    out, lse = blockwise.finalize(st)
    assert abs(out[0, 0] - g["output"]) <= half
    o_dense, lse_dense = dense.attention(np.ones((1, 1, 1)),
                                         np.array([1.0, 2, 3, 0]).reshape(1, 4, 1),
                                         np.array([1.0, 2, 3, 4]).reshape(1, 4, 1),
                                         np.array([9]), np.arange(4), False, 1.0)
    assert abs(out[0, 0] - o_dense[0, 0, 0]) < 1e-15
    assert abs(lse[0] - lse_dense[0, 0]) < 1e-15


def test_shift_invariance():
    """'Ring Attention Math Deep', online-softmax identity: any constant works."""
    q, ks, vs = _rand_case(21, 2, 4, 8, 6)
    scale = 0.3
    for causal in (False, True):
        o0, l0 = _dense_rank(dense.attention, q, ks, vs, 2, range(4), causal, scale)
        mx = float(np.max(np.abs(q))) * float(np.max(np.abs(np.concatenate(ks, 1)))) * 6 * scale
        for shift in (0.0, mx + 5.0, mx - 5.0, -mx):
            o1, l1 = _dense_rank(dense.attention, q, ks, vs, 2, range(4), causal, scale, shift)
            assert np.allclose(o1, o0, rtol=1e-12, atol=1e-13)
            assert np.allclose(l1, l0, rtol=1e-12, atol=1e-13)


def _blockwise_rank(q, ks, vs, i, order, causal, scale, skip=True):
    H, c, _ = q.shape
    qp = dense.ring_positions(i, c)
    outs, lses = [], []
    for h in range(H):
        st = blockwise.empty_state(c, vs[0].shape[2])
        for j in order:
            if causal and skip and j > i:
                continue
            s = (q[h] @ ks[j][h].T) * scale
            allowed = None
            if causal:
                allowed = dense.ring_positions(j, c)[None, :] <= qp[:, None]
            st = blockwise.fold_block(st, s, vs[j][h], allowed)
        o, lse = blockwise.finalize(st)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


def test_blockwise_any_order_equals_dense():
    """Online folding in any block order lands on the dense answer."""
    P = 5
    q, ks, vs = _rand_case(31, 2, P, 6, 4)
    rng = np.random.default_rng(0)
    for causal in (False, True):
        od, ld = _dense_rank(dense.attention, q, ks, vs, 3, range(P), causal, 0.5)
        for _ in range(20):
            order = rng.permutation(P)
            ob, lb = _blockwise_rank(q, ks, vs, 3, order, causal, 0.5)
            assert np.allclose(ob, od, rtol=1e-12, atol=1e-13)
            assert np.allclose(lb, ld, rtol=1e-12, atol=1e-13)


def test_merge_of_partitions_equals_dense():
    """Merging two partial states over a split of the blocks gives the dense
    answer; the empty state is the identity."""
    P = 6
    q, ks, vs = _rand_case(41, 1, P, 5, 3)
    rng = np.random.default_rng(1)
    c = 5
    qp = dense.ring_positions(4, c)
    for causal in (False, True):
        od, ld = _dense_rank(dense.attention, q, ks, vs, 4, range(P), causal, 0.7)
        for _ in range(10):
            perm = rng.permutation(P)
            cut = int(rng.integers(0, P + 1))
            parts = [perm[:cut], perm[cut:]]
            states = []
            for part in parts:
                st = blockwise.empty_state(c, 3)
                for j in part:
                    s = (q[0] @ ks[j][0].T) * 0.7
                    allowed = (dense.ring_positions(j, c)[None, :] <= qp[:, None]) if causal else None
                    st = blockwise.fold_block(st, s, vs[j][0], allowed)
                states.append(st)
            merged = blockwise.merge(states[0], states[1])
            o, lse = blockwise.finalize(merged)
            assert np.allclose(o, od[0], rtol=1e-12, atol=1e-13)
            assert np.allclose(lse, ld[0], rtol=1e-12, atol=1e-13)
        empty = blockwise.empty_state(c, 3)
        m2 = blockwise.merge(states[0], empty)
        assert np.array_equal(m2.m, states[0].m) and np.array_equal(m2.l, states[0].l)
        assert np.array_equal(m2.o, states[0].o)


def test_causal_skip_of_future_blocks():
    """Causal rank i: blocks j > i contribute nothing, so the dense answer over
    all blocks equals the dense answer over blocks j <= i, and the blockwise
    model that skips them agrees."""
    P = 4
    q, ks, vs = _rand_case(51, 2, P, 7, 5)
    for i in range(P):
        oa, la = _dense_rank(dense.attention, q, ks, vs, i, range(P), True, 0.4)
        ob, lb = _dense_rank(dense.attention, q, ks, vs, i, range(i + 1), True, 0.4)
        assert np.allclose(oa, ob, rtol=1e-14, atol=1e-15)
        assert np.allclose(la, lb, rtol=1e-14, atol=1e-15)
        order = [(i - s) % P for s in range(P)]
        oc, lc = _blockwise_rank(q, ks, vs, i, order, True, 0.4, skip=True)
        assert np.allclose(oc, oa, rtol=1e-12, atol=1e-13)
        assert np.allclose(lc, la, rtol=1e-12, atol=1e-13)


def test_empty_rows():
    """A row with no allowed key: O = 0, LSE = -inf (no NaN)."""
    q, ks, vs = _rand_case(61, 1, 2, 3, 2)
    o, lse = dense.attention(q, ks[1], vs[1], dense.ring_positions(0, 3),
                             dense.ring_positions(1, 3), True, 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    o, lse = dense.attention(q, ks[1][:, :0], vs[1][:, :0], dense.ring_positions(0, 3),
                             np.zeros(0, dtype=np.int64), False, 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 0.0, 3.3895313892515355e38, 9.183549615799121e-41]
    assert dense.bf16_bits_to_f64(bits).tolist() == want


# ------------------------------------------------ planted mistakes -------------

MUTATIONS = {
    "dropped scale": ("(q[h, r0:r1] @ k[h].T) * scale", "(q[h, r0:r1] @ k[h].T)"),
    "exclusive causal": ("k_pos[None, :] <= q_pos[r0:r1, None]", "k_pos[None, :] < q_pos[r0:r1, None]"),
    "reversed causal": ("k_pos[None, :] <= q_pos[r0:r1, None]", "k_pos[None, :] >= q_pos[r0:r1, None]"),
    "wrong sign of shift": ("np.exp(s - c[:, None])", "np.exp(s + c[:, None])"),
    "dropped shift in LSE": ("row_lse = c + np.log(l)", "row_lse = np.log(l)"),
    "no normalisation": ("o = num / l[:, None]", "o = num"),
    "keys reversed": ("(q[h, r0:r1] @ k[h].T)", "(q[h, r0:r1] @ k[h][::-1].T)"),
    "values reversed": ("num = w @ v[h]", "num = w @ v[h][::-1]"),
    "transposed head": ("(q[h, r0:r1] @ k[h].T)", "(q[h, r0:r1] @ k[-1 - h].T)"),
    "ln vs log2": ("row_lse = c + np.log(l)", "row_lse = c + np.log2(l)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    src = open(dense.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor missing: {old}"
    ns = {}
    exec(compile(src.replace(old, new), "mutant_dense", "exec"), ns)
    mutant = ns["attention"]
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake '{name}'"
