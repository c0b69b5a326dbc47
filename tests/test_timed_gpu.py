"""GPU: the timed entry points (ra_step_timed, ra_bwd_step_timed).

Their results are exactly those of the untimed forms (bit-identical), their
events bracket the step's kernels, and a stop event orders another stream
after the kernel it is bound to, which is what the ring's staging protocol
relies on when it uses a timed step's stop event as the buffer-free edge.
"""
import sys

import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.hip_events import Event
from ring_attention_block_amd.ring import RingEmulator, ZigzagRing, zigzag_blocks

from _helpers import gen_blocks, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.lib()


def _blocks(wl, roles_blocks):
    host = gen_blocks(wl, roles_blocks)
    return {key: to_device(x, wl) for key, x in host.items()}


STEP_CASES = [(2, 128, 300, "bf16"), (3, 64, 129, "bf16"), (1, 64, 200, "f32"), (2, 128, 64, "f32")]


@pytest.mark.parametrize("heads,d,rows,dtype", STEP_CASES)
@pytest.mark.parametrize("kv_block", [0, 1])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_timed_step_is_bit_identical(heads, d, rows, dtype, kv_block, flags):
    wl = synth.Workload(f"timed_{dtype}_h{heads}_d{d}_c{rows}", 700 + rows + d, heads, d, rows, 2,
                        dtype, True, (0, 1))
    dev = _blocks(wl, [(synth.ROLE_Q, 1), (synth.ROLE_K, 0), (synth.ROLE_V, 0), (synth.ROLE_K, 1),
                       (synth.ROLE_V, 1)])
    q, k, v = dev[(synth.ROLE_Q, 1)], dev[(synth.ROLE_K, kv_block)], dev[(synth.ROLE_V, kv_block)]
    _say(f"  timed step {wl.name} j={kv_block} flags={flags}")
    results = []
    for timed in (False, True):
        st = _lib.State(1, heads, rows, d)
        _lib.state_init(st)
        _lib.step(st, q, *[dev[(r, 0)] for r in (synth.ROLE_K, synth.ROLE_V)], 1, 0, 2, True, wl.scale)
        o = torch.full(st.o.shape, float("nan"), device="cuda")
        lse = torch.full(st.m.shape, float("nan"), device="cuda")
        ev = (Event(timing=True), Event(timing=True)) if timed else (None, None)
        _lib.step(st, q, k, v, 1, kv_block, 2, True, wl.scale, flags=flags, o_out=o, lse_out=lse,
                  start=ev[0], stop=ev[1])
        torch.cuda.synchronize()
        if timed:
            assert ev[0].elapsed_time(ev[1]) > 0
        results.append([t.clone() for t in (st.m, st.l, st.o, o, lse)])
    for a, b in zip(*results):
        assert torch.equal(a.nan_to_num(7.0), b.nan_to_num(7.0))


def test_timed_skip_and_empty_record_events():
    wl = synth.Workload("timed_skip_bf16", 760, 2, 128, 96, 2, "bf16", True, (0, 1))
    dev = _blocks(wl, [(synth.ROLE_Q, 0), (synth.ROLE_K, 1), (synth.ROLE_V, 1)])
    st = _lib.State(1, 2, 96, 128)
    o = torch.full(st.o.shape, 5.0, device="cuda")
    lse = torch.full(st.m.shape, 5.0, device="cuda")
    e0, e1 = Event(timing=True), Event(timing=True)
    case = _lib.step(st, dev[(synth.ROLE_Q, 0)], dev[(synth.ROLE_K, 1)], dev[(synth.ROLE_V, 1)], 0, 1,
                     2, True, wl.scale, flags=_lib.RA_STEP_FRESH | _lib.RA_STEP_FINALIZE, o_out=o,
                     lse_out=lse, start=e0, stop=e1)
    torch.cuda.synchronize()
    assert case == _lib.RA_CASE_SKIP
    assert e0.elapsed_time(e1) >= 0
    assert not o.any() and bool(torch.isneginf(lse).all())
    # skipped backward block: both events recorded, nothing else
    z = torch.zeros(1, 2, 96, 128, device="cuda")
    r = torch.zeros(1, 2, 96, device="cuda")
    e2, e3 = Event(timing=True), Event(timing=True)
    _lib.bwd_step(dev[(synth.ROLE_Q, 0)], dev[(synth.ROLE_Q, 0)], r, r, dev[(synth.ROLE_K, 1)],
                  dev[(synth.ROLE_V, 1)], z, z.clone(), z.clone(), 0, 1, 2, True, wl.scale,
                  start=e2, stop=e3)
    torch.cuda.synchronize()
    assert e2.elapsed_time(e3) >= 0


def test_stop_event_orders_another_stream():
    """A stream that waits on a timed step's stop event runs after the kernel
    has ended: an event recorded there after the wait is later than the stop
    timestamp."""
    wl = synth.Workload("timed_order_bf16", 770, 8, 128, 4096, 2, "bf16", True, (0, 1))
    dev = _blocks(wl, [(synth.ROLE_Q, 1), (synth.ROLE_K, 0), (synth.ROLE_V, 0)])
    st = _lib.State(1, 8, 4096, 128)
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        e0, e1, after = Event(timing=True), Event(timing=True), Event(timing=True)
        _lib.step(st, dev[(synth.ROLE_Q, 1)], dev[(synth.ROLE_K, 0)], dev[(synth.ROLE_V, 0)], 1, 0, 2,
                  True, wl.scale, stream=a, flags=_lib.RA_STEP_FRESH, start=e0, stop=e1)
        e1.wait(b)
        after.record(b)
        torch.cuda.synchronize()
        kernel_ms, gap_ms = e0.elapsed_time(e1), e1.elapsed_time(after)
        _say(f"  full step {kernel_ms * 1e3:.1f} us, waiting stream {gap_ms * 1e3:.1f} us after it")
        assert kernel_ms > 0.005 and gap_ms >= 0


def _rings(wl, rank):
    return _blocks(wl, [(synth.ROLE_Q, rank)] + [(r, j) for j in range(wl.blocks)
                                                 for r in (synth.ROLE_K, synth.ROLE_V)])


@pytest.mark.parametrize("rank", [3, 7])
def test_timed_ring_is_bit_identical(rank):
    """The fused contiguous ring with a pair of timing events on every step
    (and the stop events as the buffer-free edges) gives the untimed ring's
    outputs exactly."""
    wl = synth.Workload("timed_ring_bf16", 780, 8, 128, 1024, 8, "bf16", True, tuple(range(8)))
    dev = _rings(wl, rank)
    q = dev[(synth.ROLE_Q, rank)]
    src = lambda j: (dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)])
    emu = RingEmulator(q.shape, q.dtype)
    st = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
    outs = []
    for timed in (False, True, True):
        out = (torch.empty(st.o.shape, device="cuda"), torch.empty(st.m.shape, device="cuda"))
        timers = [] if timed else None
        emu.run(st, q, src, rank, wl.blocks, True, wl.scale, step_timers=timers, finalize_out=out)
        torch.cuda.synchronize()
        if timed:
            assert len(timers) == rank + 1
            assert all(a.elapsed_time(b) > 0 for _, a, b in timers)
        outs.append(out)
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_timed_zigzag_ring_is_bit_identical():
    ranks, rank = 4, 1
    wl = synth.Workload("timed_zz_bf16", 790, 4, 128, 512, 2 * ranks, "bf16", True,
                        tuple(range(2 * ranks)))
    dev = _blocks(wl, [(synth.ROLE_Q, b) for b in zigzag_blocks(rank, ranks)] +
                  [(r, j) for j in range(2 * ranks) for r in (synth.ROLE_K, synth.ROLE_V)])
    qs = [dev[(synth.ROLE_Q, b)] for b in zigzag_blocks(rank, ranks)]

    def source(j):
        a, b = zigzag_blocks(j, ranks)
        return (dev[(synth.ROLE_K, a)], dev[(synth.ROLE_K, b)], dev[(synth.ROLE_V, a)],
                dev[(synth.ROLE_V, b)])

    ring = ZigzagRing(qs[0].shape, qs[0].dtype)
    states = [_lib.State(1, wl.heads, wl.rows, wl.head_dim) for _ in range(2)]
    results = []
    for timed in (False, True):
        outs = [(torch.empty(st.o.shape, device="cuda"), torch.empty(st.m.shape, device="cuda"))
                for st in states]
        timers = [] if timed else None
        ring.run(states, qs, source, rank, ranks, True, wl.scale, step_timers=timers,
                 finalize_outs=outs)
        torch.cuda.synchronize()
        if timed:
            assert timers and all(a.elapsed_time(b) > 0 for _, a, b in timers)
        results.append(outs)
    for (o0, l0), (o1, l1) in zip(*results):
        assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_timed_backward_ring_is_bit_identical():
    """The contiguous backward ring (dK, dV travelling with their blocks) with
    timed steps gives the untimed ring's gradients exactly (the bf16 backward
    kernels use no atomics)."""
    P, rank = 4, 3
    wl = synth.Workload("timed_bwd_bf16", 800, 4, 128, 512, P, "bf16", True, tuple(range(P)))
    dev = _blocks(wl, [(synth.ROLE_Q, rank), (synth.ROLE_DO, rank)] +
                  [(r, j) for j in range(P) for r in (synth.ROLE_K, synth.ROLE_V)])
    q, do = dev[(synth.ROLE_Q, rank)], dev[(synth.ROLE_DO, rank)]
    shape = q.shape
    st = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
    fwd = RingEmulator(shape, q.dtype)
    fwd.run(st, q, lambda j: (dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)]), rank, P, True, wl.scale)
    o, lse = _lib.finalize(st, torch.float32, fwd.compute)
    delta = _lib.bwd_prepare(o, do, stream=fwd.compute)
    torch.cuda.synchronize()
    bwd = RingEmulator(shape, q.dtype, extra_specs=[(shape, torch.float32), (shape, torch.float32)])
    results = []
    for timed in (False, True):
        dq = torch.zeros(shape, device="cuda")
        grads = {j: (torch.zeros(shape, device="cuda"), torch.zeros(shape, device="cuda"))
                 for j in range(P)}
        source = lambda j: (dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)], *grads[j])
        timers = [] if timed else None
        bwd.run_backward(q, do, lse, delta, dq, source, rank, P, True, wl.scale, step_timers=timers)
        torch.cuda.synchronize()
        if timed:
            assert len(timers) == rank + 1 and all(a.elapsed_time(b) > 0 for _, a, b in timers)
        results.append([dq] + [t for j in range(P) for t in grads[j]])
    for a, b in zip(*results):
        assert torch.equal(a, b)
