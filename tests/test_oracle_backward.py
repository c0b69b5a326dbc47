"""Pins of the fp64 backward oracle (oracle/backward.py) to mathematics.

The pages give no gradient formulas ("Ring Attention：把超长序列沿设备环流动",
section "Backward 需要让梯度也沿环传播", only says what accumulates where and
that the saved log-sum-exp lets each block recompute its probabilities), so
the oracle is the chain rule of the dense forward, pinned here by:
  * central finite differences of L = sum(dO * O) through the dense forward
    oracle, on tiny inputs, causal and not;
  * torch autograd in float64 on the CPU (a library routine);
  * invariants: the key gradients sum to zero, the value gradients sum to the
    output gradients of the rows, equal value rows give zero dQ and dK;
  * the ring's split: summing the per-block contribution (probabilities
    recomputed from the saved LSE) over any partition of the keys gives the
    dense gradients;
and each planted mistake in the oracle's source must fail at least one pin.
"""
import numpy as np
import pytest

from oracle import backward, dense


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(h, r, n, d, seed, causal, offset=0):
    q, do = _rand((h, r, d), seed), _rand((h, r, d), seed + 1)
    k, v = _rand((h, n, d), seed + 2), _rand((h, n, d), seed + 3)
    qp = np.arange(offset, offset + r)
    kp = np.arange(n)
    return q, k, v, do, qp, kp, causal, 1.0 / np.sqrt(d)


def pin_finite_differences(bwd, blk):
    for causal in (False, True):
        q, k, v, do, qp, kp, c, scale = _case(2, 5, 7, 3, 11, causal, offset=2)
        dq, dk, dv = bwd(q, k, v, do, qp, kp, c, scale)

        def loss(q_, k_, v_):
            o, _ = dense.attention(q_, k_, v_, qp, kp, c, scale)
            return float(np.sum(do * o))

        eps = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
                a_p = [xp if nm == name else a for nm, a in zip("qkv", args)]
                a_m = [xm if nm == name else a for nm, a in zip("qkv", args)]
                num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * eps)
            assert np.max(np.abs(num - g)) < 1e-7, (name, causal, np.max(np.abs(num - g)))


def pin_torch_autograd(bwd, blk):
    torch = pytest.importorskip("torch")
    for causal in (False, True):
        q, k, v, do, qp, kp, c, scale = _case(3, 17, 23, 8, 5, causal, offset=4)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = (tq @ tk.transpose(-1, -2)) * scale
        mask = torch.tensor(backward._mask(qp, kp, c))
        s = s.masked_fill(~mask, float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        o.backward(torch.tensor(do))
        dq, dk, dv = bwd(q, k, v, do, qp, kp, c, scale)
        for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.max(np.abs(got - want.numpy())) < 1e-12


def pin_invariants(bwd, blk):
    for causal in (False, True):
        q, k, v, do, qp, kp, c, scale = _case(2, 30, 40, 16, 21, causal, offset=10)
        dq, dk, dv = bwd(q, k, v, do, qp, kp, c, scale)
        # every row here sees at least one key: sum_k P_ik = 1 and sum_k dS_ik = 0
        assert np.max(np.abs(dk.sum(axis=1))) < 1e-10
        assert np.max(np.abs(dv.sum(axis=1) - do.sum(axis=1))) < 1e-10
        # equal value rows: O is that row whatever P is, so dQ = dK = 0
        v_eq = np.broadcast_to(v[:, :1], v.shape).copy()
        dq0, dk0, _ = bwd(q, k, v_eq, do, qp, kp, c, scale)
        assert np.max(np.abs(dq0)) < 1e-12 and np.max(np.abs(dk0)) < 1e-12
        assert np.max(np.abs(dq)) > 1e-3   # and not trivially zero otherwise


def pin_blockwise_split(bwd, blk):
    for causal in (False, True):
        q, k, v, do, qp, kp, c, scale = _case(2, 24, 48, 8, 31, causal, offset=24)
        o, lse = dense.attention(q, k, v, qp, kp, c, scale)
        d_row = backward.row_dot(do, o)
        dq_ref, dk_ref, dv_ref = bwd(q, k, v, do, qp, kp, c, scale)
        rng = np.random.default_rng(3)
        cuts = np.sort(rng.choice(np.arange(1, 48), size=4, replace=False))
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for a, b in zip(np.r_[0, cuts], np.r_[cuts, 48]):
            gq, gk, gv = blk(q, k[:, a:b], v[:, a:b], do, lse, d_row, qp, kp[a:b], c, scale)
            dq += gq
            dk[:, a:b] += gk
            dv[:, a:b] += gv
        for got, want in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
            assert np.max(np.abs(got - want)) < 1e-12


PINS = [pin_finite_differences, pin_torch_autograd, pin_invariants, pin_blockwise_split]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_oracle_pins(pin):
    pin(backward.attention_backward, backward.block_backward)


def test_empty_rows_contribute_nothing():
    q, k, v, do, qp, kp, _, scale = _case(1, 4, 6, 4, 3, True, offset=0)
    kp = kp + 10                       # every key after every query: nothing allowed
    dq, dk, dv = backward.attention_backward(q, k, v, do, qp, kp, True, scale)
    assert not dq.any() and not dk.any() and not dv.any()
    lse = np.full((1, 4), -np.inf)
    gq, gk, gv = backward.block_backward(q, k, v, do, lse, np.zeros((1, 4)), qp, kp, True, scale)
    assert not gq.any() and not gk.any() and not gv.any()


MUTATIONS = {
    "missing D": ("ds = p * (dp - d_row[:, None])", "ds = p * dp"),
    "dV from Q": ("dv[h] = p.T @ do[h]", "dv[h] = p.T @ q[h]"),
    "dropped scale on dQ": ("dq[h] = scale * (ds @ k[h])", "dq[h] = (ds @ k[h])"),
    "dK from dS not transposed": ("dk[h] = scale * (ds.T @ q[h])", "dk[h] = scale * (ds.T @ do[h])"),
    "dP with V not transposed": ("dp = do[h] @ v[h].T", "dp = do[h] @ k[h].T"),
    "block: lse sign": ("s - lse[h][:, None]", "s + lse[h][:, None]"),
    "block: D sign": ("ds = p * (dp - d_row[h][:, None])", "ds = p * (dp + d_row[h][:, None])"),
    "block: dK uses dO": ("dk[h] = scale * (ds.T @ q[h])\n    return dq, dk, dv\n\n\ndef forward_for_backward",
                          "dk[h] = scale * (ds.T @ do[h])\n    return dq, dk, dv\n\n\ndef forward_for_backward"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    src = open(backward.__file__).read().replace("from .dense import attention",
                                                  "from oracle.dense import attention")
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor missing: {old}"
    ns = {"__name__": "mutant_backward"}
    exec(compile(src.replace(old, new, 1), "mutant_backward", "exec"), ns)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ns["attention_backward"], ns["block_backward"])
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake '{name}'"
