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


def A(k):
    """The k-th of a set of aligned, mutually far apart fake device addresses
    (64 GiB apart, so that no tensor of these tests overlaps another)."""
    return (1 << 40) + k * (1 << 36)


def _state(rows=128, d=128, m=A(0), l=A(1), o=A(2), batch=1, heads=2):
    return _lib.RaState(batch, heads, rows, d, m, l, o)


def _step(L, st, q=A(3), k=A(4), v=A(5), dtype=_lib.RA_BF16, kv_rows=None, i=1, j=0, P=2,
          causal=1, scale=0.125):
    kv = st.rows if kv_rows is None else kv_rows
    return L.ra_step(ctypes.byref(st), q, k, v, dtype, kv, i, j, P, causal, scale, None)


def test_step_rejects_before_enqueue(L):
    st = _state()
    assert L.ra_step(None, A(3), A(4), A(5), 1, 128, 1, 0, 2, 1, 0.1, None) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, _state(d=96)) == _lib.RA_ERR_UNSUPPORTED
    assert b"head_dim" in L.ra_last_error()
    assert _step(L, _state(d=0)) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, _state(rows=-1)) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, kv_rows=64) == _lib.RA_ERR_UNSUPPORTED   # causal needs equal blocks
    assert b"causal" in L.ra_last_error()
    assert _step(L, st, kv_rows=-1, causal=0) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, kv_rows=64, causal=0, k=0) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, kv_rows=64, causal=0, k=A(4) + 4) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, i=2, P=2) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, j=-1) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, causal=3) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, dtype=7) == _lib.RA_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _step(L, st, scale=bad) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, q=0) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, v=A(5) + 8) == _lib.RA_ERR_INVALID_ARG
    assert b"aligned" in L.ra_last_error()
    # bf16 blocks: below 2^31 bytes per (batch, head) (head_dim 128: fewer than 2^23 rows)
    assert _step(L, _state(rows=1 << 23)) == _lib.RA_ERR_UNSUPPORTED
    assert b"2^31" in L.ra_last_error()
    assert _step(L, _state(m=0)) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, _state(o=A(2) + 4)) == _lib.RA_ERR_INVALID_ARG


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
    assert b"overlap" in L.ra_last_error()
    assert L.ra_lse_merge(None, ctypes.byref(a), None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_finalize(ctypes.byref(a), A(6), 5, None, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_finalize(ctypes.byref(a), A(6) + 2, 0, None, None) == _lib.RA_ERR_INVALID_ARG
    for parts in (0, -1, 3):
        assert L.ra_merge_finalize(ctypes.byref(_state(batch=2)), parts, A(6), 0, None,
                                   None) == _lib.RA_ERR_INVALID_ARG
    assert b"divide" in L.ra_last_error()
    assert L.ra_merge_finalize(ctypes.byref(_state(batch=2)), 2, A(6), 5, None,
                               None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_merge_finalize(ctypes.byref(_state(batch=2)), 2, A(6) + 4, 0, None,
                               None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_merge_finalize(None, 1, A(6), 0, None, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_stage_block(FAKE, None, 16, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_stage_block(FAKE, FAKE + 8, 16, None) == _lib.RA_ERR_INVALID_ARG
    assert b"overlap" in L.ra_last_error()
    assert L.ra_stage_block(FAKE, FAKE + 4096 + 8, 16, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_stage_block(FAKE, FAKE + 4096, 24, None) == _lib.RA_ERR_INVALID_ARG
    assert b"aligned" in L.ra_last_error()
    assert L.ra_state_init(None, None) == _lib.RA_ERR_INVALID_ARG


def test_stage_block_ex_rejects(L):
    """ra_stage_block_ex: the same argument rules as ra_stage_block, and no
    flag bit but RA_STAGE_ALONE."""
    alone = _lib.RA_STAGE_ALONE
    assert L.ra_stage_block_ex(None, None, 0, alone, None) == _lib.RA_OK
    assert L.ra_stage_block_ex(FAKE, FAKE + 4096, 16, 2, None) == _lib.RA_ERR_INVALID_ARG
    assert b"flags" in L.ra_last_error()
    assert L.ra_stage_block_ex(FAKE, None, 16, alone, None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_stage_block_ex(FAKE, FAKE + 8, 16, alone, None) == _lib.RA_ERR_INVALID_ARG
    assert b"overlap" in L.ra_last_error()
    assert L.ra_stage_block_ex(FAKE, FAKE + 4096, 24, alone, None) == _lib.RA_ERR_INVALID_ARG
    assert b"aligned" in L.ra_last_error()


BWD_NAMES = ("q", "dout", "lse", "delta", "k", "v", "dq", "dk", "dv")
BWD_ADDR = {name: A(3 + n) for n, name in enumerate(BWD_NAMES)}


def _bwd(L, q=BWD_ADDR["q"], dout=BWD_ADDR["dout"], lse=BWD_ADDR["lse"], delta=BWD_ADDR["delta"],
         k=BWD_ADDR["k"], v=BWD_ADDR["v"], dtype=_lib.RA_BF16, dq=BWD_ADDR["dq"],
         dk=BWD_ADDR["dk"], dv=BWD_ADDR["dv"], i=1, j=0, P=2, causal=1, scale=0.125, rows=128,
         d=128):
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
    for name in BWD_NAMES:
        assert _bwd(L, **{name: 0}) == _lib.RA_ERR_INVALID_ARG, name
        assert _bwd(L, **{name: BWD_ADDR[name] + 4}) == _lib.RA_ERR_INVALID_ARG, name
        assert b"aligned" in L.ra_last_error()
    # a causal future block and an empty block enqueue nothing
    assert _bwd(L, i=0, j=1) == _lib.RA_OK
    assert _bwd(L, rows=0, q=0, dout=0, lse=0, delta=0, k=0, v=0, dq=0, dk=0, dv=0) == _lib.RA_OK

    prep = lambda **kw: L.ra_bwd_prepare(1, 2, kw.get("rows", 128), kw.get("d", 128),
                                         kw.get("o", A(0)), kw.get("ot", _lib.RA_F32),
                                         kw.get("dout", A(1)), kw.get("dt", _lib.RA_BF16),
                                         kw.get("delta", A(2)), kw.get("dq", None), None)
    assert prep(d=32) == _lib.RA_ERR_UNSUPPORTED
    assert prep(ot=4) == _lib.RA_ERR_INVALID_ARG
    assert prep(dt=4) == _lib.RA_ERR_INVALID_ARG
    for n, name in enumerate(("o", "dout", "delta")):
        assert prep(**{name: 0}) == _lib.RA_ERR_INVALID_ARG, name
        assert prep(**{name: A(n) + 8}) == _lib.RA_ERR_INVALID_ARG, name
    assert prep(dq=A(3) + 4) == _lib.RA_ERR_INVALID_ARG
    assert prep(rows=0, o=0, dout=0, delta=0) == _lib.RA_OK


def test_step_ex_rejects_before_enqueue(L):
    st = _state()
    def ex(flags, o=A(6), ot=_lib.RA_F32, lse=A(7), **kw):
        args = dict(q=A(3), k=A(4), v=A(5), i=1, j=0, P=2, causal=1)
        args.update(kw)
        return L.ra_step_ex(ctypes.byref(st), args["q"], args["k"], args["v"], _lib.RA_BF16, st.rows,
                            args["i"], args["j"], args["P"], args["causal"], 0.125, flags, o, ot, lse, None)
    assert ex(8) == _lib.RA_ERR_INVALID_ARG
    assert b"ra_step_ex" in L.ra_last_error() and b"flags" in L.ra_last_error()
    # the query broadcast flag is accepted (a skipped block enqueues nothing)
    assert ex(_lib.RA_STEP_Q_BROADCAST, i=0, j=1) == _lib.RA_OK
    assert ex(_lib.RA_STEP_Q_BROADCAST | _lib.RA_STEP_FRESH, q=0) == _lib.RA_ERR_INVALID_ARG
    assert ex(_lib.RA_STEP_FINALIZE, ot=3) == _lib.RA_ERR_INVALID_ARG
    assert ex(_lib.RA_STEP_FINALIZE, o=A(6) + 8) == _lib.RA_ERR_INVALID_ARG
    assert ex(_lib.RA_STEP_FINALIZE, lse=A(7) + 2) == _lib.RA_ERR_INVALID_ARG   # lse_out: 4-byte aligned
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
        args = dict(q=A(3), k=A(4), v=A(5), i=1, j=0, P=2, causal=1, scale=0.125)
        args.update(kw)
        return L.ra_step_timed(ctypes.byref(st), args["q"], args["k"], args["v"], _lib.RA_BF16,
                               st.rows, args["i"], args["j"], args["P"], args["causal"],
                               args["scale"], flags, A(6), _lib.RA_F32, A(7), bogus, bogus, None)
    assert timed(flags=8) == _lib.RA_ERR_INVALID_ARG
    assert b"ra_step_timed" in L.ra_last_error() and b"flags" in L.ra_last_error()
    assert timed(i=2) == _lib.RA_ERR_INVALID_ARG
    assert timed(q=0) == _lib.RA_ERR_INVALID_ARG
    assert timed(scale=0.0) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_step_timed(None, A(3), A(4), A(5), _lib.RA_BF16, 128, 1, 0, 2, 1, 0.125, 0, None,
                           _lib.RA_F32, None, bogus, bogus, None) == _lib.RA_ERR_INVALID_ARG
    # no events, nothing to fold: OK without any HIP call
    assert L.ra_step_timed(ctypes.byref(st), A(3), A(4), A(5), _lib.RA_BF16, st.rows, 0, 1, 2, 1,
                           0.125, 0, None, _lib.RA_F32, None, None, None, None) == _lib.RA_OK

    def bwd(**kw):
        args = dict(d=128, q=BWD_ADDR["q"], i=1, j=0, scale=0.125)
        args.update(kw)
        ad = BWD_ADDR
        return L.ra_bwd_step_timed(1, 2, 128, args["d"], args["q"], ad["dout"], ad["lse"],
                                   ad["delta"], ad["k"], ad["v"], _lib.RA_BF16, ad["dq"], ad["dk"],
                                   ad["dv"], args["i"], args["j"], 2, 1, args["scale"], bogus, bogus,
                                   None)
    assert bwd(d=96) == _lib.RA_ERR_UNSUPPORTED
    assert b"ra_bwd_step_timed" in L.ra_last_error()
    assert bwd(q=BWD_ADDR["q"] + 4) == _lib.RA_ERR_INVALID_ARG
    assert bwd(i=3) == _lib.RA_ERR_INVALID_ARG
    assert bwd(scale=float("nan")) == _lib.RA_ERR_INVALID_ARG
    ad = BWD_ADDR
    assert L.ra_bwd_step_timed(1, 2, 128, 128, ad["q"], ad["dout"], ad["lse"], ad["delta"], ad["k"],
                               ad["v"], _lib.RA_BF16, ad["dq"], ad["dk"], ad["dv"], 0, 1, 2, 1,
                               0.125, None, None, None) == _lib.RA_OK


# ------------------------------------------------------------ overlapping buffers
# Sizes at the default shapes: a state of 1 x 2 x 128 rows, head_dim 128, has
# m, l of 1 KiB and o of 128 KiB; bf16 q, k, v of 64 KiB.

def test_state_parts_must_be_disjoint(L):
    assert _step(L, _state(l=A(0) + 512)) == _lib.RA_ERR_INVALID_ARG   # l inside m
    assert b"state m" in L.ra_last_error() and b"overlap" in L.ra_last_error()
    assert _step(L, _state(m=A(2) + 128 * 1024 - 16)) == _lib.RA_ERR_INVALID_ARG   # m at o's tail
    assert L.ra_state_init(ctypes.byref(_state(o=A(1))), None) == _lib.RA_ERR_INVALID_ARG
    # adjacent but disjoint ranges are accepted (a skipped block enqueues nothing)
    ok = _state(m=A(0), l=A(0) + 1024, o=A(0) + 2048)
    assert _step(L, ok, i=0, j=1) == _lib.RA_OK


def test_step_rejects_state_overlapping_inputs(L):
    st = _state()
    assert _step(L, st, q=A(2) + 64 * 1024) == _lib.RA_ERR_INVALID_ARG   # q inside state o
    assert b"state o" in L.ra_last_error() and b"q" in L.ra_last_error()
    assert _step(L, st, k=A(0)) == _lib.RA_ERR_INVALID_ARG
    assert _step(L, st, v=A(1) - 16) == _lib.RA_ERR_INVALID_ARG           # v's tail on l
    # read-only inputs may share memory
    assert _step(L, st, k=A(4), v=A(4), i=0, j=1) == _lib.RA_OK
    # q just past the end of state o is fine (nothing enqueued for a skip)
    assert _step(L, st, q=A(2) + 128 * 1024, i=0, j=1) == _lib.RA_OK


def test_finalizing_step_rejects_outputs_overlapping(L):
    st = _state()
    def ex(o, lse):
        return L.ra_step_ex(ctypes.byref(st), A(3), A(4), A(5), _lib.RA_BF16, st.rows, 1, 0, 2, 1,
                            0.125, _lib.RA_STEP_FINALIZE, o, _lib.RA_F32, lse, None)
    assert ex(A(2), A(7)) == _lib.RA_ERR_INVALID_ARG          # o_out on the state's o
    assert b"o_out" in L.ra_last_error()
    assert ex(A(6), A(6) + 4096) == _lib.RA_ERR_INVALID_ARG   # lse_out inside o_out
    assert ex(A(6), A(3)) == _lib.RA_ERR_INVALID_ARG          # lse_out on q


def test_merge_finalize_reject_overlapping_ranges(L):
    a = _state()
    b = _state(m=A(6), l=A(7), o=A(8))
    # src's o starting inside dst's o (not at the same base)
    b_o = _state(m=A(6), l=A(7), o=A(2) + 4096)
    assert L.ra_lse_merge(ctypes.byref(a), ctypes.byref(b_o), None) == _lib.RA_ERR_INVALID_ARG
    assert b"dst o" in L.ra_last_error() and b"src o" in L.ra_last_error()
    # src's m overlapping dst's l
    b_m = _state(m=A(1) + 512, l=A(7), o=A(8))
    assert L.ra_lse_merge(ctypes.byref(a), ctypes.byref(b_m), None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_finalize(ctypes.byref(a), A(2) + 16, 0, A(9), None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_finalize(ctypes.byref(a), A(9), 0, A(0), None) == _lib.RA_ERR_INVALID_ARG
    assert L.ra_finalize(ctypes.byref(a), A(9), 1, A(9) + 32 * 1024, None) == _lib.RA_ERR_INVALID_ARG
    a2 = _state(batch=2)
    assert L.ra_merge_finalize(ctypes.byref(a2), 2, A(0), 0, A(9), None) == _lib.RA_ERR_INVALID_ARG
    assert b"overlap" in L.ra_last_error()


def test_bwd_rejects_overlapping_gradients_and_inputs(L):
    ad = BWD_ADDR
    assert _bwd(L, dk=ad["dv"]) == _lib.RA_ERR_INVALID_ARG               # dk == dv would sum both
    assert b"dk" in L.ra_last_error() and b"dv" in L.ra_last_error()
    assert _bwd(L, dq=ad["dk"] + 4096) == _lib.RA_ERR_INVALID_ARG
    assert _bwd(L, dv=ad["q"] + 16) == _lib.RA_ERR_INVALID_ARG
    assert _bwd(L, dq=ad["lse"]) == _lib.RA_ERR_INVALID_ARG
    # inputs may share memory (q is k in self-attention of one block)
    assert _bwd(L, k=ad["q"], i=0, j=1) == _lib.RA_OK
    prep = lambda o=A(0), dout=A(1), delta=A(2), dq=A(3): L.ra_bwd_prepare(
        1, 2, 128, 128, o, _lib.RA_F32, dout, _lib.RA_BF16, delta, dq, None)
    assert prep(dq=A(0) + 16) == _lib.RA_ERR_INVALID_ARG                 # dq on o
    assert prep(dq=A(1)) == _lib.RA_ERR_INVALID_ARG                      # dq on dout
    assert prep(delta=A(3) + 512) == _lib.RA_ERR_INVALID_ARG             # delta inside dq
    assert prep(delta=A(0)) == _lib.RA_ERR_INVALID_ARG                   # delta on o
    assert b"overlap" in L.ra_last_error()


def _staged(L, st, copies, n=None, q=A(3), k=A(4), v=A(5), flags=0, o_out=None, lse_out=None,
            i=1, j=0, causal=1):
    arr = (_lib.RaCopy * max(1, len(copies)))(*[_lib.RaCopy(d, s, b) for d, s, b in copies])
    n = len(copies) if n is None else n
    return L.ra_step_staged(ctypes.byref(st), q, k, v, _lib.RA_BF16, st.rows, i, j, 2, causal, 0.125,
                            flags, o_out, _lib.RA_F32, lse_out, arr if copies or n else None, n,
                            None, None, None)


def test_step_staged_rejects_before_enqueue(L):
    st = _state()
    big = 1 << 20
    ok_copy = (A(8), A(9), big)
    bad = _lib.RA_ERR_INVALID_ARG
    assert _staged(L, st, [ok_copy] * 3) == bad                       # more than RA_MAX_STEP_COPIES
    assert _staged(L, st, [], n=-1) == bad
    assert L.ra_step_staged(ctypes.byref(st), A(3), A(4), A(5), 1, 128, 1, 0, 2, 1, 0.125, 0, None, 0,
                            None, None, 1, None, None, None) == bad   # NULL copies
    assert _staged(L, st, [(0, A(9), big)]) == bad                    # NULL dst
    assert _staged(L, st, [(A(8) + 8, A(9), big)]) == bad             # misaligned
    assert _staged(L, st, [(A(8), A(9), big + 8)]) == bad             # not a multiple of 16
    assert b"16" in L.ra_last_error()
    assert _staged(L, st, [(A(8), A(9), 1 << 31)]) == bad             # 2^31 bytes
    assert _staged(L, st, [(A(8), A(8) + 4096, big)]) == bad          # dst overlaps its src
    assert b"overlap" in L.ra_last_error()
    assert _staged(L, st, [ok_copy, (A(8) + 64, A(10), 4096)]) == bad  # two destinations overlap
    assert _staged(L, st, [ok_copy, (A(10), A(8), 4096)]) == bad       # dst is another copy's src
    assert _staged(L, st, [(A(4), A(9), 4096)]) == bad                # dst over k
    assert _staged(L, st, [(A(3) + 4096, A(9), 4096)]) == bad         # dst over q
    assert _staged(L, st, [(A(2), A(9), 4096)]) == bad                # dst over the state
    assert _staged(L, st, [(A(8), A(2), 4096)]) == bad                # src over the state (written)
    assert _staged(L, st, [(A(8), A(6), 4096)], flags=_lib.RA_STEP_FINALIZE, o_out=A(6)) == bad
    assert b"o_out" in L.ra_last_error()
    # the step's own checks still apply
    assert _staged(L, st, [ok_copy], q=A(3) + 8) == bad


def _strided(L, st, rs, kvs, q=A(3), k=A(4), v=A(5), kv_rows=None, i=1, j=0, P=2, causal=1,
             flags=0, o_out=None, lse_out=None):
    kv = st.rows if kv_rows is None else kv_rows
    return L.ra_step_strided(ctypes.byref(st), rs, q, k, v, _lib.RA_BF16, kv, kvs, i, j, P, causal,
                             0.125, flags, o_out, _lib.RA_F32, lse_out, None, 0, None, None, None)


def test_strided_step_rejects_before_enqueue(L):
    st = _state(rows=128)
    assert _strided(L, st, 127, 128) == _lib.RA_ERR_INVALID_ARG      # row stride below rows
    assert b"row_stride" in L.ra_last_error()
    assert _strided(L, st, 256, 100, kv_rows=128, causal=0) == _lib.RA_ERR_INVALID_ARG
    assert b"kv_row_stride" in L.ra_last_error()
    assert _strided(L, st, -1, 128) == _lib.RA_ERR_INVALID_ARG
    assert _strided(L, st, 128, -5) == _lib.RA_ERR_INVALID_ARG
    # extents that overlap: m of two heads 2^30 rows apart (2^32 bytes) reaches l
    far = _state(rows=128, m=A(0), l=A(0) + (1 << 31), o=A(2), heads=2)
    assert _strided(L, far, 1 << 30, 128) == _lib.RA_ERR_INVALID_ARG
    assert b"state m and state l overlap" in L.ra_last_error()
    # a strided state that folds nothing cannot take FRESH / FINALIZE (the state kernels are packed)
    assert _strided(L, st, 256, 128, i=0, j=1, flags=_lib.RA_STEP_FRESH) == _lib.RA_ERR_UNSUPPORTED
    assert _strided(L, st, 256, 128, kv_rows=0, causal=0,
                    flags=_lib.RA_STEP_FINALIZE) == _lib.RA_ERR_UNSUPPORTED
    # the same calls at the packed stride are the ordinary skip / empty no-ops ... minus the
    # state kernels, which would launch: only plain no-op calls here
    assert _strided(L, st, 128, 128, i=0, j=1) == _lib.RA_OK
    assert _strided(L, st, 256, 128, i=0, j=1) == _lib.RA_OK
    assert _strided(L, _state(rows=0, m=0, l=0, o=0), 0, 0, q=0, k=0, v=0) == _lib.RA_OK
    # the checks of ra_step_staged still apply
    assert _strided(L, _state(d=96), 128, 128) == _lib.RA_ERR_UNSUPPORTED
    assert _strided(L, st, 256, 256, q=A(3) + 4) == _lib.RA_ERR_INVALID_ARG
