"""Randomised checks of the C ABI's host-side validation (no GPU needed).

Each example builds a valid, non-skipped, non-empty ra_step_ex call on fake
device addresses, then breaks it with one to three mutations, each of which a
host check must reject (a head size other than 64 or 128, negative sizes,
indices out of range, misaligned or NULL tensors, an invalid scale, causal
value, dtype, output dtype or flag, unequal blocks under the causal mask, an
output overlapping an input).  The call must return RA_ERR_INVALID_ARG or
RA_ERR_UNSUPPORTED with a message: never RA_OK and never RA_ERR_HIP, i.e.
nothing reaches a launch.  Every generated case is invalid by construction,
so no call can enqueue work on any machine.
"""
import ctypes
import math
import os

import pytest

from ring_attention_block_amd import _lib

hypothesis = pytest.importorskip("hypothesis")
st = hypothesis.strategies


def A(k):
    """Aligned fake device addresses, 64 GiB apart: never dereferenced."""
    return (1 << 40) + k * (1 << 36)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libra.so is not built (python -m ring_attention_block_amd.build)")
    return _lib.lib()


BREAKERS = ["head_dim", "neg_size", "q_block", "kv_block", "blocks", "misalign_q", "misalign_k",
            "misalign_v", "null_q", "null_k", "misalign_m", "misalign_o", "scale", "causal",
            "dtype", "flags", "causal_unequal", "out_dtype", "misalign_out", "out_overlaps_q"]


@st.composite
def broken_call(draw):
    c = dict(
        batch=draw(st.integers(1, 3)), heads=draw(st.integers(1, 4)),
        rows=draw(st.integers(1, 300)), d=draw(st.sampled_from([64, 128])),
        dtype=draw(st.sampled_from([_lib.RA_F32, _lib.RA_BF16])),
        P=draw(st.integers(1, 8)), causal=draw(st.integers(0, 1)),
        scale=draw(st.floats(1e-3, 2.0)),
        flags=draw(st.sampled_from([0, _lib.RA_STEP_FRESH, _lib.RA_STEP_FINALIZE,
                                    _lib.RA_STEP_FRESH | _lib.RA_STEP_FINALIZE])),
        m=A(0), l=A(1), o=A(2), q=A(3), k=A(4), v=A(5), o_out=A(6), lse_out=A(7),
        out_dtype=draw(st.sampled_from([_lib.RA_F32, _lib.RA_BF16])))
    # a launched step: i >= j (full or diagonal) under the causal mask
    c["i"] = draw(st.integers(0, c["P"] - 1))
    c["j"] = draw(st.integers(0, c["i"]))
    c["kv_rows"] = c["rows"] if c["causal"] else draw(st.integers(1, 300))
    for b in draw(st.lists(st.sampled_from(BREAKERS), min_size=1, max_size=3, unique=True)):
        if b == "head_dim":
            c["d"] = draw(st.sampled_from([-64, 0, 16, 32, 96, 192, 256]))
        elif b == "neg_size":
            c[draw(st.sampled_from(["batch", "heads", "rows"]))] = -draw(st.integers(1, 5))
        elif b == "q_block":
            c["i"] = draw(st.sampled_from([-1, c["P"], c["P"] + 3]))
        elif b == "kv_block":
            c["j"] = draw(st.sampled_from([-1, c["P"], c["P"] + 3]))
        elif b == "blocks":
            c["P"] = draw(st.integers(-3, 0))
        elif b in ("misalign_q", "misalign_k", "misalign_v"):
            c[b[-1]] += draw(st.sampled_from([2, 4, 8]))
        elif b in ("null_q", "null_k"):
            c[b[-1]] = 0
        elif b == "misalign_m":
            c["m"] += draw(st.sampled_from([1, 2]))
        elif b == "misalign_o":
            c["o"] += draw(st.sampled_from([2, 4, 8]))
        elif b == "scale":
            c["scale"] = draw(st.sampled_from([0.0, -0.5, math.inf, -math.inf, math.nan]))
        elif b == "causal":
            c["causal"] = draw(st.sampled_from([-1, 2, 7]))
        elif b == "dtype":
            c["dtype"] = draw(st.sampled_from([-1, 2, 9]))
        elif b == "flags":
            c["flags"] |= draw(st.sampled_from([8, 16, 1 << 20]))
        elif b == "causal_unequal":
            c["causal"] = 1
            c["kv_rows"] = c["rows"] + draw(st.integers(1, 64))
        elif b == "out_dtype":
            c["flags"] |= _lib.RA_STEP_FINALIZE
            c["out_dtype"] = draw(st.sampled_from([-1, 2, 5]))
        elif b == "misalign_out":
            c["flags"] |= _lib.RA_STEP_FINALIZE
            c["o_out"] += draw(st.sampled_from([2, 4, 8]))
        elif b == "out_overlaps_q":
            c["flags"] |= _lib.RA_STEP_FINALIZE
            c["o_out"] = c["q"]
    return c


@hypothesis.settings(max_examples=400, deadline=None, derandomize=True)
@hypothesis.given(broken_call())
def test_broken_step_ex_is_rejected_on_the_host(L, c):
    state = _lib.RaState(c["batch"], c["heads"], c["rows"], c["d"], c["m"], c["l"], c["o"])
    rc = L.ra_step_ex(ctypes.byref(state), c["q"], c["k"], c["v"], c["dtype"], c["kv_rows"], c["i"],
                      c["j"], c["P"], c["causal"], c["scale"], c["flags"], c["o_out"], c["out_dtype"],
                      c["lse_out"], None)
    assert rc in (_lib.RA_ERR_INVALID_ARG, _lib.RA_ERR_UNSUPPORTED), (rc, c)
    assert L.ra_last_error(), c


BWD_BREAKERS = ["head_dim", "neg_size", "q_block", "kv_block", "causal", "dtype", "scale",
                "misalign", "null", "dq_is_dk", "dk_is_dv", "dq_overlaps_q", "misalign_lse"]


@st.composite
def broken_bwd(draw):
    c = dict(batch=draw(st.integers(1, 3)), heads=draw(st.integers(1, 4)),
             rows=draw(st.integers(1, 300)), d=draw(st.sampled_from([64, 128])),
             dtype=draw(st.sampled_from([_lib.RA_F32, _lib.RA_BF16])),
             P=draw(st.integers(1, 8)), causal=draw(st.integers(0, 1)),
             scale=draw(st.floats(1e-3, 2.0)),
             q=A(0), dout=A(1), lse=A(2), delta=A(3), k=A(4), v=A(5), dq=A(6), dk=A(7), dv=A(8))
    c["i"] = draw(st.integers(0, c["P"] - 1))
    c["j"] = draw(st.integers(0, c["i"]))
    for b in draw(st.lists(st.sampled_from(BWD_BREAKERS), min_size=1, max_size=3, unique=True)):
        if b == "head_dim":
            c["d"] = draw(st.sampled_from([-128, 0, 32, 96, 256]))
        elif b == "neg_size":
            c[draw(st.sampled_from(["batch", "heads", "rows"]))] = -draw(st.integers(1, 5))
        elif b == "q_block":
            c["i"] = draw(st.sampled_from([-1, c["P"]]))
        elif b == "kv_block":
            c["j"] = draw(st.sampled_from([-1, c["P"]]))
        elif b == "causal":
            c["causal"] = draw(st.sampled_from([-1, 2]))
        elif b == "dtype":
            c["dtype"] = draw(st.sampled_from([-1, 2]))
        elif b == "scale":
            c["scale"] = draw(st.sampled_from([0.0, -1.0, math.inf, math.nan]))
        elif b == "misalign":
            c[draw(st.sampled_from(["q", "dout", "k", "v", "dq", "dk", "dv"]))] += draw(st.sampled_from([2, 4, 8]))
        elif b == "null":
            c[draw(st.sampled_from(["q", "dout", "lse", "delta", "k", "v", "dq", "dk", "dv"]))] = 0
        elif b == "dq_is_dk":
            c["dk"] = c["dq"]
        elif b == "dk_is_dv":
            c["dv"] = c["dk"]
        elif b == "dq_overlaps_q":
            c["dq"] = c["q"]
        elif b == "misalign_lse":
            c[draw(st.sampled_from(["lse", "delta"]))] += draw(st.sampled_from([1, 2]))
    return c


@hypothesis.settings(max_examples=300, deadline=None, derandomize=True)
@hypothesis.given(broken_bwd())
def test_broken_bwd_step_is_rejected_on_the_host(L, c):
    rc = L.ra_bwd_step(c["batch"], c["heads"], c["rows"], c["d"], c["q"], c["dout"], c["lse"],
                       c["delta"], c["k"], c["v"], c["dtype"], c["dq"], c["dk"], c["dv"], c["i"],
                       c["j"], c["P"], c["causal"], c["scale"], None)
    assert rc in (_lib.RA_ERR_INVALID_ARG, _lib.RA_ERR_UNSUPPORTED), (rc, c)
    assert L.ra_last_error(), c


STRIDE_BREAKERS = ["row_stride", "kv_row_stride", "neg_stride", "fresh_on_skip", "misalign_q",
                   "head_dim", "scale", "extent_overlap"]


@st.composite
def broken_strided(draw):
    c = dict(batch=draw(st.integers(1, 3)), heads=draw(st.integers(1, 4)),
             rows=draw(st.integers(1, 300)), d=draw(st.sampled_from([64, 128])),
             scale=draw(st.floats(1e-3, 2.0)), flags=0, causal=0, i=0, j=0, P=1,
             m=A(0), l=A(1), o=A(2), q=A(3), k=A(4), v=A(5))
    c["kv_rows"] = draw(st.integers(1, 300))
    c["rs"] = c["rows"] + draw(st.integers(0, 300))
    c["kvs"] = c["kv_rows"] + draw(st.integers(0, 300))
    for b in draw(st.lists(st.sampled_from(STRIDE_BREAKERS), min_size=1, max_size=3, unique=True)):
        if b == "row_stride":
            c["rs"] = c["rows"] - draw(st.integers(1, c["rows"]))
        elif b == "kv_row_stride":
            c["kvs"] = c["kv_rows"] - draw(st.integers(1, c["kv_rows"]))
        elif b == "neg_stride":
            c[draw(st.sampled_from(["rs", "kvs"]))] = -draw(st.integers(1, 1 << 20))
        elif b == "fresh_on_skip":
            # a causal future block folds nothing; FRESH then needs a packed state
            c.update(causal=1, kv_rows=c["rows"], kvs=max(c["kvs"], c["rows"]), i=0, j=1, P=2,
                     flags=draw(st.sampled_from([1, 2, 3])))
            c["rs"] = c["rows"] + draw(st.integers(1, 64))
        elif b == "misalign_q":
            c["q"] += draw(st.sampled_from([2, 4, 8]))
        elif b == "head_dim":
            c["d"] = draw(st.sampled_from([0, 32, 96, 256]))
        elif b == "scale":
            c["scale"] = draw(st.sampled_from([0.0, -1.0, math.inf, math.nan]))
        elif b == "extent_overlap":
            # m's extent over (batch*heads - 1) strides reaches l
            c.update(batch=1, heads=2, rs=1 << 30, l=A(0) + (1 << 31))
    return c


@hypothesis.settings(max_examples=300, deadline=None, derandomize=True)
@hypothesis.given(broken_strided())
def test_broken_strided_step_is_rejected_on_the_host(L, c):
    state = _lib.RaState(c["batch"], c["heads"], c["rows"], c["d"], c["m"], c["l"], c["o"])
    rc = L.ra_step_strided(ctypes.byref(state), c["rs"], c["q"], c["k"], c["v"], _lib.RA_BF16,
                           c["kv_rows"], c["kvs"], c["i"], c["j"], c["P"], c["causal"], c["scale"],
                           c["flags"], None, _lib.RA_F32, None, None, 0, None, None, None)
    assert rc in (_lib.RA_ERR_INVALID_ARG, _lib.RA_ERR_UNSUPPORTED), (rc, c)
    assert L.ra_last_error(), c
