"""GPU parity of the exact code path bench.py times, on every query row, and
the ring's robustness checks (extreme scores, buffer hazards, a state
checkpoint).

The benchmarked ring (bench.py) runs on its own compute stream with the init
fused into the first launched step (RA_STEP_FRESH), the finalize fused into
the last (RA_STEP_FINALIZE), and timing events bound to every step kernel's
dispatch (ra_step_timed), whose stop events also release the staging buffers.
At 32 heads x 4096 rows x head_dim 128 both the full and the diagonal step
launch 8-wavefront workgroups (32 heads x 16 query tiles of 256 rows = 512
workgroups, at least one per compute unit).

Inputs come from ring_attention_block_amd.synth, expected values from oracle/
only.  Tolerances (max abs error): fp32 inputs 1e-5 on O and LSE; bf16 inputs
with fp32 accumulation 2e-2 on O and 5e-3 on LSE.
"""
import concurrent.futures as cf
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.hip_events import Event
from ring_attention_block_amd.ring import RingEmulator, key_split_for, ring_order, split_keys, staging_for

from _helpers import assert_close, gen_blocks, oracle_rank, to_device, tol_for

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.lib()


class Inputs:
    def __init__(self, wl, rank, blocks=None):
        self.wl = wl
        blocks = list(range(wl.blocks) if blocks is None else blocks)
        jobs = [(synth.ROLE_Q, rank)] + [(r, j) for j in blocks for r in (synth.ROLE_K, synth.ROLE_V)]
        self.cache = gen_blocks(wl, jobs)
        self.q = to_device(self.cache[(synth.ROLE_Q, rank)], wl)
        self.kv = {j: (to_device(self.cache[(synth.ROLE_K, j)], wl),
                       to_device(self.cache[(synth.ROLE_V, j)], wl)) for j in blocks}

    def set_rank(self, rank):
        key = (synth.ROLE_Q, rank)
        if key not in self.cache:
            self.cache[key] = synth.block(self.wl, *key)
        self.q = to_device(self.cache[key], self.wl)


def bench_ring(inp, rank, causal, order=None, free_hook=None, out_dtype=torch.float32,
               key_split=None, staging=None):
    """One ring exactly as bench.py enqueues it: own compute stream, fused
    init and finalize, every launched step timed by events bound to its
    dispatch (drawn from a pool created beforehand); without the causal mask
    a small query block takes bench.py's key split (key_split_for) unless
    key_split is given, and the staging mode is bench.py's (staging_for)
    unless staging is given."""
    wl = inp.wl
    ks = key_split_for(wl.heads, wl.rows, wl.rows, causal) if key_split is None else key_split
    kv = inp.kv if ks == 1 else {j: (split_keys(k, ks), split_keys(v, ks)) for j, (k, v) in inp.kv.items()}
    steps = ring_order(rank, wl.blocks) if order is None else list(order)
    step_cases = [_lib.step_case(rank, j, wl.blocks, causal) for j in steps]
    launched = sum(c != _lib.RA_CASE_SKIP for c in step_cases)
    if staging is None:
        staging = staging_for(ks * wl.heads, wl.rows, wl.rows // ks, wl.head_dim,
                              step_cases.count(_lib.RA_CASE_SKIP))
    compute = torch.cuda.Stream()
    st = _lib.State(ks, wl.heads, wl.rows, wl.head_dim)
    emu = RingEmulator(kv[next(iter(kv))][0].shape, inp.q.dtype, compute_stream=compute, staging=staging)
    emu.free_hook = free_hook
    o = torch.empty((1, *st.o.shape[1:]), dtype=out_dtype, device="cuda")
    lse = torch.empty((1, *st.m.shape[1:]), dtype=torch.float32, device="cuda")
    pool = iter([Event(timing=True) for _ in range(2 * launched)])
    timers = []
    emu.run(st, inp.q, lambda j: kv[j], rank, wl.blocks, causal, wl.scale, order=order,
            step_timers=timers, timer_events=pool, finalize_out=(o, lse), key_split=ks)
    torch.cuda.synchronize()
    assert len(timers) == launched
    assert all(a.elapsed_time(b) > 0 for _, a, b in timers)
    return o, lse


def plain_ring(inp, rank, causal, order=None, out_dtype=torch.float32):
    """The same ring with separate init and finalize launches, untimed."""
    wl = inp.wl
    st = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
    emu = RingEmulator(inp.q.shape, inp.q.dtype)
    emu.run(st, inp.q, lambda j: inp.kv[j], rank, wl.blocks, causal, wl.scale, order=order)
    o, lse = _lib.finalize(st, out_dtype, emu.compute)
    torch.cuda.synchronize()
    return o, lse


def oracle_every_head(wl, rank, blocks, causal, cache, threads=16, row_block=2048):
    """oracle_rank over every head and row, as (head, block of row_block query
    rows) tasks on a thread pool (numpy releases the GIL in its products and
    exponentials; one BLAS thread each), printing progress as they finish."""
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        one_blas_thread = threadpool_limits(limits=1)   # applies now, restores on exit
    except ImportError:       # pragma: no cover
        one_blas_thread = contextlib.nullcontext()
    for key in [(synth.ROLE_Q, rank)] + [(r, j) for j in blocks for r in (synth.ROLE_K, synth.ROLE_V)]:
        if key not in cache:
            cache[key] = synth.block(wl, *key)
    tasks = [(h, r0) for h in range(wl.heads) for r0 in range(0, wl.rows, row_block)]

    def one(task):
        h, r0 = task
        rows = np.arange(r0, min(wl.rows, r0 + row_block))
        return oracle_rank(wl, rank, blocks, causal, row_sel=rows, head_sel=[h], cache=cache)

    parts = {}
    with one_blas_thread, cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futures = {ex.submit(one, t): t for t in tasks}
        for n, fut in enumerate(cf.as_completed(futures), 1):
            parts[futures[fut]] = fut.result()
            if n % max(1, len(tasks) // 8) == 0 or n == len(tasks):
                _say(f"    oracle: {n} of {len(tasks)} (head, row block) tasks")
    o = np.stack([np.concatenate([parts[(h, r0)][0][0] for r0 in range(0, wl.rows, row_block)])
                  for h in range(wl.heads)])
    lse = np.stack([np.concatenate([parts[(h, r0)][1][0] for r0 in range(0, wl.rows, row_block)])
                    for h in range(wl.heads)])
    return o, lse


def check_all(wl, o, lse, want, what, lse_slack=None):
    got_o = o[0].float().cpu().numpy()
    got_l = lse[0].cpu().numpy()
    to, tl = tol_for(wl)
    if lse_slack is not None:
        tl = tl + lse_slack
    eo = assert_close(got_o, want[0], to, f"{what} O")
    el = assert_close(got_l, want[1], tl, f"{what} LSE")
    _say(f"  {what}: every row: max|dO|={eo:.2e} max|dLSE|={el:.2e}")
    return eo, el


# --------------------------------------------------- the benchmarked path, in full

C2 = synth.WORKLOADS["causal_bf16_h32_d128_c4096_p8"]


@pytest.fixture(scope="module")
def c2_inputs():
    return Inputs(C2, 7)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rank", [7, 3, 0])
def test_bench_path_causal_h32_d128_c4096_every_row(c2_inputs, rank):
    """Ranks 7 (diagonal + 7 full blocks: the headline), 3 and 0 through the
    fused, timed ring: all 4096 rows x 32 heads against the oracle, and bit
    for bit the unfused, untimed ring."""
    inp = c2_inputs
    inp.set_rank(rank)
    _say(f"{C2.name} rank {rank}: fused timed ring")
    o, lse = bench_ring(inp, rank, True)
    o2, lse2 = plain_ring(inp, rank, True)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "fused timed ring differs from the plain ring"
    _say(f"  oracle over {rank + 1} key blocks, every row")
    want = oracle_every_head(C2, rank, list(range(rank + 1)), True, inp.cache)
    check_all(C2, o, lse, want, f"rank {rank}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rq", [1, 16, 64])
def test_bench_decode_path_every_row(c2_inputs, rq):
    """The decode step bench.py times (--decode-rows R): R query rows after the
    sequence against the workload's 8 blocks as key/value shards, each shard
    laid out as decode.splits_for chunks along the batch axis (2 at 1 and 16
    rows, 1 at 64), one fold whose dispatch carries timing events and one
    merge-and-finalize: every row and head against the oracle over all 32768
    keys."""
    from oracle import dense
    from ring_attention_block_amd.decode import ChunkedDecode, splits_for
    from _helpers import oracle_values
    inp, wl = c2_inputs, C2
    P, c = wl.blocks, wl.rows
    S = splits_for(P, wl.heads, c, rq)
    _say(f"{wl.name}: decode {rq} rows, {S} chunk(s) per shard")
    qh = synth.block(wl, synth.ROLE_Q, P, rows=rq)
    q = to_device(qh, wl)
    k = torch.cat([split_keys(inp.kv[j][0], S) for j in range(P)], dim=0)
    v = torch.cat([split_keys(inp.kv[j][1], S) for j in range(P)], dim=0)
    dec = ChunkedDecode(q.shape, P * S)
    start, stop = Event(timing=True), Event(timing=True)
    o, lse = dec.run(q, k, v, wl.scale, start=start, stop=stop)
    torch.cuda.synchronize()
    assert start.elapsed_time(stop) > 0
    to, tl = tol_for(wl)
    kp, qp = np.arange(P * c), np.full(rq, P * c)
    eo = el = 0.0
    for hh in range(wl.heads):
        want_o, want_lse = dense.attention(
            oracle_values(qh[hh:hh + 1], wl),
            np.concatenate([oracle_values(inp.cache[(synth.ROLE_K, j)][hh:hh + 1], wl) for j in range(P)], axis=1),
            np.concatenate([oracle_values(inp.cache[(synth.ROLE_V, j)][hh:hh + 1], wl) for j in range(P)], axis=1),
            qp, kp, False, wl.scale)
        eo = max(eo, assert_close(o[0, hh].cpu().numpy(), want_o[0], to, f"head {hh} O"))
        el = max(el, assert_close(lse[0, hh].cpu().numpy(), want_lse[0], tl, f"head {hh} LSE"))
    _say(f"  every row and head: max|dO|={eo:.2e} max|dLSE|={el:.2e}")


@pytest.mark.timeout(900)
def test_bench_path_longshare_d64_every_row():
    """The long-share ring bench.py times (--workload
    longshare_bf16_h16_d64_c16384_p32): rank 31 folds all 32 blocks of 16384
    keys at head_dim 64 (diagonal, then 31 full blocks) through the fused,
    timed ring with side staging; every one of the 16384 rows x 16 heads
    against the oracle over all 524288 keys."""
    wl = synth.WORKLOADS["longshare_bf16_h16_d64_c16384_p32"]
    rank = wl.ranks[-1]
    inp = Inputs(wl, rank)
    _say(f"{wl.name} rank {rank}: fused timed ring")
    o, lse = bench_ring(inp, rank, True)
    _say(f"  oracle over {wl.blocks} key blocks, every row")
    want = oracle_every_head(wl, rank, list(range(wl.blocks)), True, inp.cache)
    check_all(wl, o, lse, want, f"rank {rank}")


C3 = synth.WORKLOADS["rescale_bf16_h8_d128_c2048_p16"]


@pytest.mark.timeout(900)
def test_rescale_stress_every_row_both_orders():
    """The rescale-stress workload (+2j on every score against block j) in ring
    order (the row maximum falls at every step) and reversed (it rises at every
    step), both through the benchmarked path, on every row."""
    rank = 15
    inp = Inputs(C3, rank)
    fwd = ring_order(rank, C3.blocks)
    want = oracle_every_head(C3, rank, list(range(C3.blocks)), False, inp.cache)
    res = []
    for name, order in (("ring order", fwd), ("reversed", fwd[::-1])):
        _say(f"{C3.name} {name}")
        o, lse = bench_ring(inp, rank, False, order=order)
        check_all(C3, o, lse, want, name)
        res.append((o, lse))
    # The benchmarked ring folds each block as two key halves (the query block
    # alone would fill half the chip) and merges them at the end; the plain
    # ring folds whole blocks.  Both are within the tolerance of the oracle
    # (above) and of each other; the unsplit ring through the benchmarked path
    # is bit-identical to the plain one.
    assert key_split_for(C3.heads, C3.rows, C3.rows, False) == 2
    o2, lse2 = plain_ring(inp, rank, False, order=fwd)
    assert float((res[0][0] - o2).abs().max()) <= 2e-2 and float((res[0][1] - lse2).abs().max()) <= 5e-3
    o1, lse1 = bench_ring(inp, rank, False, order=fwd, key_split=1)
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    assert float((res[0][0] - res[1][0]).abs().max()) <= 2e-2
    assert float((res[0][1] - res[1][1]).abs().max()) <= 5e-3


# --------------------------------------------------- extreme scores

def _lse_slack(wl, want_lse):
    """fp32 cannot hold a log-sum-exp of magnitude 10^2 to 10^3 to 1e-5: the
    stored value alone carries half a unit in the last place (2^-24 |LSE|), and
    the kernels form it from a maximum and a logarithm rounded separately.  The
    fp32 workloads get 8 units in the last place of the largest |LSE| on top of
    the stated tolerance; the bf16 tolerance (5e-3) already covers them."""
    if wl.dtype != "f32":
        return None
    fin = np.isfinite(want_lse)
    return 8 * 2.0 ** -23 * float(np.max(np.abs(want_lse[fin])))


# (name, dtype, heads, head_dim, rows, P, rank, causal, spike, spike_blocks, spike_key, order)
#   order: None = ring order j = rank, rank-1, ...; "rev" = reversed.
# Score offsets of magnitude 10^2 to 10^3.  For rank 3 of 4 in ring order the
# blocks are visited 3, 2, 1, 0: block 3 first, block 1 in the middle, block 0
# last.  One-key spikes make every row dominated by a single key; a spike key
# inside the diagonal block is masked for every row before it.
EXTREME = [
    ("max_first", "bf16", 2, 128, 300, 4, 3, False, 600.0, (3,), -1, None),
    ("max_middle", "bf16", 2, 128, 300, 4, 3, False, 600.0, (1,), -1, None),
    ("max_last", "bf16", 2, 128, 300, 4, 3, False, 600.0, (0,), -1, None),
    ("causal_max_first", "bf16", 2, 128, 300, 4, 3, True, 900.0, (3,), -1, None),
    ("causal_max_middle", "bf16", 3, 64, 333, 4, 3, True, 900.0, (1,), -1, None),
    ("causal_max_last", "bf16", 2, 128, 300, 4, 3, True, 900.0, (0,), -1, None),
    ("one_key", "bf16", 2, 128, 300, 4, 3, True, 900.0, (1,), 5, None),
    ("one_key_d64", "bf16", 2, 64, 200, 3, 2, True, 900.0, (2,), 77, None),
    ("masked_spike_key", "bf16", 2, 128, 300, 4, 3, True, 900.0, (3,), 150, None),
    ("masked_spike_key_reversed", "bf16", 2, 128, 300, 4, 3, True, 900.0, (3,), 150, "rev"),
    ("large_negative_block", "bf16", 2, 128, 300, 4, 3, True, -700.0, (2,), -1, None),
    ("all_scores_large_negative", "bf16", 2, 128, 300, 4, 3, False, -500.0, (0, 1, 2, 3), -1, None),
    ("all_scores_large_positive", "bf16", 2, 64, 129, 4, 2, True, 800.0, (0, 1, 2, 3), -1, "rev"),
    # 8-wavefront workgroups (64 heads x 4 query tiles of 256 rows = 256 workgroups)
    ("w8_causal_max_middle", "bf16", 64, 128, 1024, 4, 3, True, 700.0, (1,), -1, None),
    ("w8_masked_spike_key", "bf16", 64, 128, 1024, 4, 3, True, 700.0, (3,), 600, None),
    # fp32 inputs (the general fp32 kernel)
    ("f32_max_first", "f32", 2, 64, 200, 3, 2, False, 100.0, (2,), -1, None),
    ("f32_max_last", "f32", 2, 64, 200, 3, 2, False, 100.0, (0,), -1, None),
    ("f32_causal_max_middle", "f32", 1, 128, 130, 3, 2, True, 100.0, (1,), -1, None),
    ("f32_masked_spike_key", "f32", 2, 64, 200, 3, 2, True, 100.0, (2,), 120, None),
    ("f32_one_key_reversed", "f32", 2, 64, 200, 3, 2, True, 100.0, (0,), 9, "rev"),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", EXTREME, ids=[c[0] for c in EXTREME])
def test_extreme_scores(case):
    """Online-softmax stability under scores of magnitude 10^2 to 10^3
    ("Ring Attention：把超长序列沿设备环流动", section "正确性测试应覆盖哪些边界",
    numerics): the row maximum arriving in the first, a middle or the last
    visited block, rows dominated by one key, a spike key hidden by the
    causal mask, and uniformly very negative or very positive scores.  Both
    the benchmarked (fused, timed) ring and the plain ring, against the oracle."""
    name, dtype, heads, d, rows, P, rank, causal, spike, blocks, key, order = case
    wl = synth.Workload(f"extreme_{name}", 1000 + rows + d + int(abs(spike)), heads, d, rows, P, dtype,
                        causal, (rank,), spike=spike, spike_blocks=blocks, spike_key=key)
    inp = Inputs(wl, rank)
    steps = ring_order(rank, P)
    if order == "rev":
        steps = steps[::-1]
    visible = [j for j in range(P) if not causal or j <= rank]
    want = oracle_every_head(wl, rank, visible, causal, inp.cache)
    assert np.all(np.isfinite(want[1])), "the oracle sees an empty row"
    _say(f"{wl.name}: |LSE| up to {float(np.max(np.abs(want[1]))):.1f}, order {steps}")
    slack = _lse_slack(wl, want[1])
    for label, fn in (("fused timed", bench_ring), ("plain", plain_ring)):
        o, lse = fn(inp, rank, causal, order=steps)
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), f"{label}: non-finite"
        check_all(wl, o, lse, want, f"{name} {label}", lse_slack=slack)


# --------------------------------------------------- key split

# (name, dtype, heads, head_dim, rows, P, rank, spike, spike_blocks, spike_key, key_split, order)
KSPLIT = [
    ("bf16_d128_halves", "bf16", 4, 128, 512, 3, 2, 0.0, (), -1, 2, None),
    ("bf16_d64_quarters", "bf16", 2, 64, 1024, 4, 1, 0.0, (), -1, 4, None),
    ("bf16_d128_quarters_reversed", "bf16", 3, 128, 1024, 3, 0, 0.0, (), -1, 4, "rev"),
    ("f32_d64_halves", "f32", 2, 64, 256, 3, 0, 0.0, (), -1, 2, None),
    ("f32_d128_quarters", "f32", 1, 128, 512, 2, 1, 0.0, (), -1, 4, None),
    # Score offsets of 10^2 in one visited block, and one key dominating its rows
    # from the second key half only (one partial state holds the maximum).
    ("bf16_spike_block", "bf16", 2, 128, 512, 3, 2, 600.0, (1,), -1, 2, None),
    ("bf16_one_key_second_half", "bf16", 2, 128, 512, 3, 2, 900.0, (0,), 400, 2, "rev"),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", KSPLIT, ids=[c[0] for c in KSPLIT])
def test_key_split_ring(case):
    """Without the causal mask, every visiting block folded as key_split
    ranges of keys into as many partial states (the query block broadcast to
    all of them) and merged once after the ring (ra_merge_finalize), as
    bench.py runs a small query block: every row against the oracle, and
    within tolerance of the unsplit ring."""
    name, dtype, heads, d, rows, P, rank, spike, blocks, key, ks, order = case
    wl = synth.Workload(f"ksplit_{name}", 500 + rows + d + ks, heads, d, rows, P, dtype, False, (rank,),
                        spike=spike, spike_blocks=blocks, spike_key=key)
    inp = Inputs(wl, rank)
    steps = ring_order(rank, P)
    if order == "rev":
        steps = steps[::-1]
    want = oracle_every_head(wl, rank, list(range(P)), False, inp.cache)
    _say(f"{wl.name}: key split {ks}, order {steps}")
    o, lse = bench_ring(inp, rank, False, order=steps, key_split=ks)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    check_all(wl, o, lse, want, f"{name} split {ks}", lse_slack=_lse_slack(wl, want[1]))
    o1, lse1 = bench_ring(inp, rank, False, order=steps, key_split=1)
    tol_o, tol_l = (2e-2, 5e-3) if dtype == "bf16" else (1e-5, 1e-5 + (_lse_slack(wl, want[1]) or 0.0))
    assert float((o - o1).abs().max()) <= 2 * tol_o and float((lse - lse1).abs().max()) <= 2 * tol_l


def test_key_split_caller_merge_and_rejects():
    """RingEmulator.run(key_split=2) without finalize_out leaves the two
    partial states to the caller: merging them with ra_merge_finalize gives
    the fused ring's outputs bit for bit.  A causal ring, or a state whose
    batch is not the number of ranges, is rejected before any launch."""
    wl = synth.Workload("ksplit_caller", 808, 2, 128, 512, 3, "bf16", False, (1,))
    inp = Inputs(wl, 1)
    o, lse = bench_ring(inp, 1, False, key_split=2)
    kv = {j: (split_keys(k, 2), split_keys(v, 2)) for j, (k, v) in inp.kv.items()}
    st = _lib.State(2, wl.heads, wl.rows, wl.head_dim)
    emu = RingEmulator(kv[0][0].shape, inp.q.dtype)
    emu.run(st, inp.q, lambda j: kv[j], 1, wl.blocks, False, wl.scale, key_split=2)
    o2, lse2 = _lib.merge_finalize(st, 2, torch.float32, emu.compute)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    with pytest.raises(ValueError, match="key_split"):
        emu.run(st, inp.q, lambda j: kv[j], 1, wl.blocks, True, wl.scale, key_split=2)
    with pytest.raises(ValueError, match="key_split"):
        emu.run(_lib.State(1, wl.heads, wl.rows, wl.head_dim), inp.q, lambda j: kv[j], 1, wl.blocks,
                False, wl.scale, key_split=2)


# --------------------------------------------------- buffer hazards

def _poison(tensors, stream):
    with torch.cuda.stream(stream):
        for t in tensors:
            t.fill_(float("nan"))


@pytest.mark.timeout(600)
def test_released_buffers_poisoned_change_nothing(c2_inputs):
    """The two hazards of double buffering ("Ring Attention：...", section
    "双缓冲是重叠成立的基础"): every receive buffer is filled with NaN on the
    copy stream as soon as its release is signalled, and the buffers start as
    NaN.  A step that still read a released buffer, or read a buffer before
    its block was staged, would put NaN into the output; the result must be
    bit-identical to the ring without poisoning."""
    inp = c2_inputs
    rank = 7
    inp.set_rank(rank)
    clean = bench_ring(inp, rank, True)
    # Both buffers start poisoned; the hook poisons each one again when it is
    # released (also after the last step).
    wl = inp.wl
    compute = torch.cuda.Stream()
    st = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
    emu = RingEmulator(inp.q.shape, inp.q.dtype, compute_stream=compute)
    for buf in emu.bufs:
        _poison(buf, emu.copy)
    emu.free_hook = _poison
    o = torch.empty(st.o.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(st.m.shape, dtype=torch.float32, device="cuda")
    pool = iter([Event(timing=True) for _ in range(2 * wl.blocks)])
    timers = []
    emu.run(st, inp.q, lambda j: inp.kv[j], rank, wl.blocks, True, wl.scale, step_timers=timers,
            timer_events=pool, finalize_out=(o, lse))
    torch.cuda.synchronize()
    assert torch.equal(o, clean[0]) and torch.equal(lse, clean[1])
    # the hook really ran: both buffers were released after their last use
    assert all(bool(torch.isnan(t.float()).all()) for b in emu.bufs for t in b)
    _say("  poisoned ring bit-identical to the clean ring")


@pytest.mark.timeout(600)
def test_backward_ring_poisoned_buffers_change_nothing():
    """The backward ring drains the travelling dK, dV out of each buffer before
    it is released; poisoning released buffers must change no gradient bit."""
    heads, d, rows, P = 4, 128, 640, 3
    wl = synth.Workload("bwd_poison", 77, heads, d, rows, P, "bf16", True, tuple(range(P)))
    jobs = [(r, j) for j in range(P) for r in (synth.ROLE_Q, synth.ROLE_K, synth.ROLE_V, synth.ROLE_DO)]
    host = gen_blocks(wl, jobs)
    dev = {key: to_device(x, wl) for key, x in host.items()}
    shape = dev[(synth.ROLE_Q, 0)].shape
    kv = {j: (dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)]) for j in range(P)}
    results = []
    for poison in (False, True):
        dk = {j: torch.zeros(shape, dtype=torch.float32, device="cuda") for j in range(P)}
        dv = {j: torch.zeros(shape, dtype=torch.float32, device="cuda") for j in range(P)}
        fwd = RingEmulator(shape, torch.bfloat16)
        bwd = RingEmulator(shape, torch.bfloat16, compute_stream=fwd.compute,
                           extra_specs=[(shape, torch.float32), (shape, torch.float32)])
        if poison:
            for buf in bwd.bufs:
                _poison(buf, bwd.copy)
            bwd.free_hook = _poison
        dq = {}
        for i in range(P):
            st = _lib.State(*shape)
            fwd.run(st, dev[(synth.ROLE_Q, i)], lambda j: kv[j], i, P, True, wl.scale)
            o, lse = _lib.finalize(st, torch.float32, fwd.compute)
            delta = _lib.bwd_prepare(o, dev[(synth.ROLE_DO, i)], stream=fwd.compute)
            dq[i] = torch.zeros(shape, dtype=torch.float32, device="cuda")
            bwd.run_backward(dev[(synth.ROLE_Q, i)], dev[(synth.ROLE_DO, i)], lse, delta, dq[i],
                             lambda j: (kv[j][0], kv[j][1], dk[j], dv[j]), i, P, True, wl.scale)
        torch.cuda.synchronize()
        results.append((dq, dk, dv))
    for name, a, b in zip(("dQ", "dK", "dV"), results[0], results[1]):
        for j in range(P):
            assert bool(torch.isfinite(b[j]).all()), f"{name}[{j}] not finite"
            assert torch.equal(a[j], b[j]), f"{name}[{j}] differs under poisoning"
    _say("  poisoned backward ring bit-identical")


# --------------------------------------------------- state checkpoint

@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_state_checkpoint_round_trip(dtype):
    """Half a ring, the state copied to the host, the device copy destroyed
    and restored from the host, the rest of the ring: bit-identical to the
    uninterrupted ring, and equal to the oracle."""
    heads, d, rows, P, rank = (4, 128, 1000, 6, 5) if dtype == "bf16" else (2, 64, 200, 6, 5)
    wl = synth.Workload(f"ckpt_{dtype}", 31 + rows, heads, d, rows, P, dtype, True, (rank,))
    inp = Inputs(wl, rank)
    order = ring_order(rank, P)
    ref = plain_ring(inp, rank, True)
    st = _lib.State(1, heads, rows, d)
    emu = RingEmulator(inp.q.shape, inp.q.dtype)
    emu.run(st, inp.q, lambda j: inp.kv[j], rank, P, True, wl.scale, order=order[:3])
    torch.cuda.synchronize()
    saved = [t.cpu().clone() for t in (st.m, st.l, st.o)]
    for t in (st.m, st.l, st.o):
        t.fill_(float("nan"))
    for t, h in zip((st.m, st.l, st.o), saved):
        t.copy_(h)
    emu.run(st, inp.q, lambda j: inp.kv[j], rank, P, True, wl.scale, order=order[3:], init=False)
    o, lse = _lib.finalize(st, torch.float32, emu.compute)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])
    want = oracle_every_head(wl, rank, list(range(rank + 1)), True, inp.cache)
    check_all(wl, o, lse, want, f"checkpointed {dtype} ring")
