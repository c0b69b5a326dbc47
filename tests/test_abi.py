"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before enqueuing."""
import ctypes
import os
import re

import pytest

from ring_attention_block_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "ra.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libra.so is not built (python -m ring_attention_block_amd.build)")
    return _lib.lib()


def test_header_matches_binding_exports():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    assert L.ra_status_string(0) == b"RA_OK"
    assert L.ra_status_string(-1) == b"RA_ERR_INVALID_ARG"
    assert L.ra_status_string(-2) == b"RA_ERR_UNSUPPORTED"
    assert L.ra_status_string(-3) == b"RA_ERR_HIP"


@pytest.mark.parametrize("P", [1, 2, 5, 8])
def test_step_case_table(L, P):
    for i in range(P):
        for j in range(P):
            assert L.ra_step_case(i, j, P, 0) == _lib.RA_CASE_FULL
            want = _lib.RA_CASE_SKIP if j > i else (_lib.RA_CASE_DIAG if j == i else _lib.RA_CASE_FULL)
            assert L.ra_step_case(i, j, P, 1) == want


def test_step_case_rejects(L):
    assert L.ra_step_case(0, 0, 0, 1) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_step_case(3, 0, 3, 1) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_step_case(0, -1, 3, 1) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_step_case(0, 0, 3, 2) == _lib.RA_ERR_INVALID_ARG
    assert b"causal" in L.ra_last_error()


FAKE = 1 << 20   # an aligned non-NULL address; never dereferenced by a rejected call


def _state(rows=128, d=128, m=FAKE, l=FAKE, o=FAKE, batch=1, heads=2):
    return _lib.RaState(batch, heads, rows, d, m, l, o)


def _step(L, st, q=FAKE, k=FAKE, v=FAKE, dtype=_lib.RA_BF16, kv_rows=None, i=1, j=0, P=2,
          causal=1, scale=0.125):
    kv = st.rows if kv_rows is None else kv_rows
    return L.ra_step(ctypes.byref(st), q, k, v, dtype, kv, i, j, P, causal, scale, None)


def test_step_rejects_before_enqueue(L):
    st = _state()
    assert L.ra_step(None, FAKE, FAKE, FAKE, 1, 128, 1, 0, 2, 1, 0.1, None) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, _state(d=96)) == _lib.RA_ERR_UNSUPPORTED
    assert b"head_dim" in L.ra_last_error()
    assert _step(L, _state(d=0)) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, _state(rows=-1)) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, kv_rows=64) == _lib.RA_ERR_UNSUPPORTED   # causal needs equal blocks
    assert b"causal" in L.ra_last_error()
    assert _step(L, st, kv_rows=-1, causal=0) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, kv_rows=64, causal=0, k=0) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, kv_rows=64, causal=0, k=FAKE + 4) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, i=2, P=2) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, j=-1) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, causal=3) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, dtype=7) == _lib.RA_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _step(L, st, scale=bad) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, q=0) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, v=FAKE + 8) == _lib.RA_ERR_INVALID_ARG
    assert b"aligned" in L.ra_last_error()
    # bf16 blocks: below 2^31 bytes per (batch, head) (head_dim 128: fewer than 2^23 rows)
    assert _step(L, _state(rows=1 << 23)) == _lib.RA_ERR_UNSUPPORTED
    assert b"2^31" in L.ra_last_error()
    assert _step(L, _state(m=0)) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, _state(o=FAKE + 4)) == _lib.RA_ERR_INVALID_ARG


def test_skip_and_empty_enqueue_nothing(L):
    # A causal future block and an empty state return OK without any HIP call,
    # so they succeed even where no GPU exists.
    assert _step(L, _state(), i=0, j=1, P=2) == _lib.RA_OK
    assert L.ra_last_error() == b""
    empty = _state(rows=0, m=0, l=0, o=0)
    assert _step(L, empty, q=0, k=0, v=0) == _lib.RA_OK
    # an empty key/value block (non-causal) folds nothing; k and v may be NULL
    assert _step(L, _state(), kv_rows=0, causal=0, k=0, v=0) == _lib.RA_OK
    assert L.ra_state_init(ctypes.byref(empty), None) == _lib.RA_OK
    assert L.ra_finalize(ctypes.byref(empty), None, 0, None, None) == _lib.RA_OK
    assert L.ra_merge_finalize(ctypes.byref(empty), 1, None, 0, None, None) == _lib.RA_OK
    assert L.ra_lse_merge(ctypes.byref(empty), ctypes.byref(_state(rows=0, m=0, l=0, o=0)), None) == 0
    assert L.ra_stage_block(None, None, 0, None) == _lib.RA_OK


def test_merge_finalize_stage_reject(L):
    a, b = _state(), _state(rows=64)
    assert L.ra_lse_merge(ctypes.byref(a), ctypes.byref(b), None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_lse_merge(ctypes.byref(a), ctypes.byref(_state()), None) == _lib.RA_ERR_INVALID_ARG
    assert b"alias" in L.ra_last_error()
    assert L.ra_lse_merge(None, ctypes.byref(a), None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_finalize(ctypes.byref(a), FAKE, 5, None, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_finalize(ctypes.byref(a), FAKE + 2, 0, None, None) == _lib.RA_ERR_INVALID_ARG
    for parts in (0, -1, 3):
        assert L.ra_merge_finalize(ctypes.byref(_state(batch=2)), parts, FAKE, 0, None,
                                   None) == _lib.RA_ERR_INVALID_ARG
    assert b"divide" in L.ra_last_error()
    assert L.ra_merge_finalize(ctypes.byref(_state(batch=2)), 2, FAKE, 5, None,
                               None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_merge_finalize(ctypes.byref(_state(batch=2)), 2, FAKE + 4, 0, None,
                               None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_merge_finalize(None, 1, FAKE, 0, None, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_stage_block(FAKE, None, 16, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_stage_block(FAKE, FAKE + 8, 16, None) == _lib.RA_ERR_INVALID_ARG
    assert b"overlap" in L.ra_last_error()
    assert L.ra_stage_block(FAKE, FAKE + 4096 + 8, 16, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_stage_block(FAKE, FAKE + 4096, 24, None) == _lib.RA_ERR_INVALID_ARG
    assert b"aligned" in L.ra_last_error()
    assert L.ra_state_init(None, None) == _lib.RA_ERR_INVALID_ARG


def _bwd(L, q=FAKE, dout=FAKE, lse=FAKE, delta=FAKE, k=FAKE, v=FAKE, dtype=_lib.RA_BF16,
         dq=FAKE, dk=FAKE, dv=FAKE, i=1, j=0, P=2, causal=1, scale=0.125, rows=128, d=128):
    return L.ra_bwd_step(1, 2, rows, d, q, dout, lse, delta, k, v, dtype, dq, dk, dv, i, j, P,
                         causal, scale, None)


def test_bwd_rejects_before_enqueue(L):
    assert _bwd(L, d=96) == _lib.RA_ERR_UNSUPPORTED
    assert b"ra_bwd_step" in L.ra_last_error() and b"head_dim" in L.ra_last_error()
    assert _bwd(L, rows=-1) == _lib.RA_ERR_INVALID_ARG
    assert _bwd(L, i=2, P=2) == _lib.RA_ERR_INVALID_ARG
    assert _bwd(L, causal=2) == _lib.RA_ERR_INVALID_ARG
    assert _bwd(L, dtype=9) == _lib.RA_ERR_INVALID_ARG
    assert _bwd(L, rows=1 << 23) == _lib.RA_ERR_UNSUPPORTED
    for bad in (0.0, -0.5, float("inf"), float("nan")):
        assert _bwd(L, scale=bad) == _lib.RA_ERR_INVALID_ARG
    for name in ("q", "dout", "lse", "delta", "k", "v", "dq", "dk", "dv"):
        assert _bwd(L, **{name: 0}) == _lib.RA_ERR_INVALID_ARG, name
        assert _bwd(L, **{name: FAKE + 4}) == _lib.RA_ERR_INVALID_ARG, name
        assert b"aligned" in L.ra_last_error()
    # a causal future block and an empty block enqueue nothing
    assert _bwd(L, i=0, j=1) == _lib.RA_OK
    assert _bwd(L, rows=0, q=0, dout=0, lse=0, delta=0, k=0, v=0, dq=0, dk=0, dv=0) == _lib.RA_OK

    prep = lambda **kw: L.ra_bwd_prepare(1, 2, kw.get("rows", 128), kw.get("d", 128),
                                         kw.get("o", FAKE), kw.get("ot", _lib.RA_F32),
                                         kw.get("dout", FAKE), kw.get("dt", _lib.RA_BF16),
                                         kw.get("delta", FAKE), kw.get("dq", None), None)
    assert prep(d=32) == _lib.RA_ERR_UNSUPPORTED
    assert prep(ot=4) == _lib.RA_ERR_INVALID_ARG
    assert prep(dt=4) == _lib.RA_ERR_INVALID_ARG
    for name in ("o", "dout", "delta"):
        assert prep(**{name: 0}) == _lib.RA_ERR_INVALID_ARG, name
        assert prep(**{name: FAKE + 8}) == _lib.RA_ERR_INVALID_ARG, name
    assert prep(dq=FAKE + 4) == _lib.RA_ERR_INVALID_ARG
    assert prep(rows=0, o=0, dout=0, delta=0) == _lib.RA_OK


def test_step_ex_rejects_before_enqueue(L):
    st = _state()
    def ex(flags, o=FAKE, ot=_lib.RA_F32, lse=FAKE, **kw):
        args = dict(q=FAKE, k=FAKE, v=FAKE, i=1, j=0, P=2, causal=1)
        args.update(kw)
        return L.ra_step_ex(ctypes.byref(st), args["q"], args["k"], args["v"], _lib.RA_BF16, st.rows,
                            args["i"], args["j"], args["P"], args["causal"], 0.125, flags, o, ot, lse, None)
    assert ex(8) == _lib.RA_ERR_INVALID_ARG
    assert b"ra_step_ex" in L.ra_last_error() and b"flags" in L.ra_last_error()
    # the query broadcast flag is accepted (a skipped block enqueues nothing)
    assert ex(_lib.RA_STEP_Q_BROADCAST, i=0, j=1) == _lib.RA_OK
    assert ex(_lib.RA_STEP_Q_BROADCAST | _lib.RA_STEP_FRESH, q=0) == _lib.RA_ERR_INVALID_ARG
    assert ex(_lib.RA_STEP_FINALIZE, ot=3) == _lib.RA_ERR_INVALID_ARG
    assert ex(_lib.RA_STEP_FINALIZE, o=FAKE + 8) == _lib.RA_ERR_INVALID_ARG
    assert ex(_lib.RA_STEP_FINALIZE, lse=FAKE + 4) == _lib.RA_ERR_INVALID_ARG
    assert ex(_lib.RA_STEP_FRESH, q=0) == _lib.RA_ERR_INVALID_ARG
    assert ex(3, i=2) == _lib.RA_ERR_INVALID_ARG
    # flags 0 on a skipped block: nothing enqueued, as ra_step
    assert ex(0, i=0, j=1) == _lib.RA_OK


def test_timed_entries_reject_before_enqueue(L):
    # The timed entry points check exactly as their untimed forms; on an error
    # nothing is enqueued and the events are not touched (invalid handles here).
    st = _state()
    bogus = ctypes.c_void_p(FAKE)
    def timed(flags=0, **kw):
        args = dict(q=FAKE, k=FAKE, v=FAKE, i=1, j=0, P=2, causal=1, scale=0.125)
        args.update(kw)
        return L.ra_step_timed(ctypes.byref(st), args["q"], args["k"], args["v"], _lib.RA_BF16,
                               st.rows, args["i"], args["j"], args["P"], args["causal"],
                               args["scale"], flags, FAKE, _lib.RA_F32, FAKE, bogus, bogus, None)
    assert timed(flags=8) == _lib.RA_ERR_INVALID_ARG
    assert b"ra_step_timed" in L.ra_last_error() and b"flags" in L.ra_last_error()
    assert timed(i=2) == _lib.RA_ERR_INVALID_ARG
    assert timed(q=0) == _lib.RA_ERR_INVALID_ARG
    assert timed(scale=0.0) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_step_timed(None, FAKE, FAKE, FAKE, _lib.RA_BF16, 128, 1, 0, 2, 1, 0.125, 0, None,
                           _lib.RA_F32, None, bogus, bogus, None) == _lib.RA_ERR_INVALID_ARG
    # no events, nothing to fold: OK without any HIP call
    assert L.ra_step_timed(ctypes.byref(st), FAKE, FAKE, FAKE, _lib.RA_BF16, st.rows, 0, 1, 2, 1,
                           0.125, 0, None, _lib.RA_F32, None, None, None, None) == _lib.RA_OK

    def bwd(**kw):
        args = dict(d=128, q=FAKE, i=1, j=0, scale=0.125)
        args.update(kw)
        return L.ra_bwd_step_timed(1, 2, 128, args["d"], args["q"], FAKE, FAKE, FAKE, FAKE, FAKE,
                                   _lib.RA_BF16, FAKE, FAKE, FAKE, args["i"], args["j"], 2, 1,
                                   args["scale"], bogus, bogus, None)
    assert bwd(d=96) == _lib.RA_ERR_UNSUPPORTED
    assert b"ra_bwd_step_timed" in L.ra_last_error()
    assert bwd(q=FAKE + 4) == _lib.RA_ERR_INVALID_ARG
    assert bwd(i=3) == _lib.RA_ERR_INVALID_ARG
    assert bwd(scale=float("nan")) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_bwd_step_timed(1, 2, 128, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, _lib.RA_BF16,
                               FAKE, FAKE, FAKE, 0, 1, 2, 1, 0.125, None, None, None) == _lib.RA_OK
