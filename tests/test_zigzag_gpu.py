"""GPU parity of the zigzag partition: ZigzagRing through the C ABI against
the fp64 CPU oracle.

Under the zigzag partition ("Ring Attention Paper Breakdown: Blockwise
Distributed Transformers for Near-Infinite Context", section 5) rank i holds
pieces i and 2P-1-i of a sequence cut into 2P pieces.  The oracle is the dense
definition at those pieces' global positions against every key piece; inputs
come from ring_attention_block_amd.synth, expected values from oracle/ only.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.ring import ZigzagRing, zigzag_blocks

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


def run_zigzag(sub, rank, ranks, causal, cache):
    """Resident pieces of `sub` (the zigzag sub-block workload), one ring of
    `rank`; returns the finalized (O, LSE) of the rank's two pieces."""
    jobs = [(synth.ROLE_Q, b) for b in zigzag_blocks(rank, ranks)]
    jobs += [(r, b) for b in range(2 * ranks) for r in (synth.ROLE_K, synth.ROLE_V)]
    missing = [j for j in jobs if j not in cache]
    cache.update(gen_blocks(sub, missing))
    dev = {key: to_device(cache[key], sub) for key in jobs}
    qs = [dev[(synth.ROLE_Q, b)] for b in zigzag_blocks(rank, ranks)]

    def source(j):
        a, b = zigzag_blocks(j, ranks)
        return (dev[(synth.ROLE_K, a)], dev[(synth.ROLE_K, b)],
                dev[(synth.ROLE_V, a)], dev[(synth.ROLE_V, b)])

    states = [_lib.State(1, sub.heads, sub.rows, sub.head_dim) for _ in range(2)]
    ring = ZigzagRing(qs[0].shape, qs[0].dtype)
    ring.run(states, qs, source, rank, ranks, causal, sub.scale)
    outs = [_lib.finalize(st, torch.float32, ring.compute) for st in states]
    torch.cuda.synchronize()
    return outs


def check_rank(sub, rank, ranks, causal, cache, rows=None):
    outs = run_zigzag(sub, rank, ranks, causal, cache)
    to, tl = tol_for(sub)
    for piece, (o, lse) in zip(zigzag_blocks(rank, ranks), outs):
        want_o, want_lse = oracle_rank(sub, piece, range(2 * ranks), causal, row_sel=rows,
                                       cache=cache)
        got_o, got_lse = o[0].cpu().numpy(), lse[0].cpu().numpy()
        if rows is not None:
            got_o, got_lse = got_o[:, rows], got_lse[:, rows]
        what = f"{sub.name} causal={causal} rank {rank} piece {piece}"
        eo = assert_close(got_o, want_o, to, what + " O")
        el = assert_close(got_lse, want_lse, tl, what + " LSE")
        _say(f"  {what}: max|dO|={eo:.2e} max|dLSE|={el:.2e}")


SMALL = [
    # (heads, head_dim, rows per rank, ranks, dtype): pieces of rows/2, ragged tails
    (2, 128, 400, 3, "bf16"),
    (1, 64, 128, 4, "f32"),
    (3, 64, 258, 2, "bf16"),
    (2, 128, 1024, 4, "bf16"),
]


@pytest.mark.parametrize("heads,d,rows,P,dtype", SMALL)
@pytest.mark.parametrize("causal", [True, False])
def test_zigzag_every_rank(heads, d, rows, P, dtype, causal):
    wl = synth.Workload(f"zz_{dtype}_h{heads}_d{d}_c{rows}_p{P}", 200 + rows + d, heads, d, rows,
                        P, dtype, causal, tuple(range(P)))
    sub = synth.zigzag_workload(wl)
    cache = {}
    for rank in range(P):
        _say(f"{sub.name} causal={causal} rank={rank}")
        check_rank(sub, rank, P, causal, cache)


@pytest.mark.timeout(900)
def test_zigzag_headline_shape_sampled_rows():
    """The headline shape (32 heads, d = 128, 4096 tokens per rank, 8 ranks)
    under the zigzag partition, ranks 0 and 7, on 64 sampled rows per piece."""
    wl = synth.WORKLOADS["causal_bf16_h32_d128_c4096_p8"]
    sub = synth.zigzag_workload(wl)
    rows = synth.sample_rows(wl.seed, sub.rows, 64)
    cache = {}
    for rank in (0, 7):
        _say(f"{sub.name} rank={rank}")
        check_rank(sub, rank, wl.blocks, True, cache, rows=rows)


@pytest.mark.parametrize("heads,d,rows,P,dtype", [(2, 128, 400, 3, "bf16"), (1, 64, 128, 4, "f32"),
                                                 (2, 128, 1024, 2, "bf16")])
@pytest.mark.parametrize("causal", [True, False])
def test_zigzag_backward_all_ranks(heads, d, rows, P, dtype, causal):
    """Every rank's zigzag forward ring, then every rank's zigzag backward ring
    (the dK, dV of each sub-block travel with it), against the dense gradients
    of the whole sequence ("Ring Attention：把超长序列沿设备环流动", section
    "Backward 需要让梯度也沿环传播"); tolerance as in test_backward_gpu.py."""
    from oracle import backward
    from _helpers import oracle_values
    wl = synth.Workload(f"zzb_{dtype}_h{heads}_d{d}_c{rows}_p{P}", 300 + rows + d, heads, d, rows,
                        P, dtype, causal, tuple(range(P)))
    sub = synth.zigzag_workload(wl)
    n = 2 * P
    host = gen_blocks(sub, [(r, b) for b in range(n)
                            for r in (synth.ROLE_Q, synth.ROLE_K, synth.ROLE_V, synth.ROLE_DO)])
    dev = {key: to_device(x, sub) for key, x in host.items()}
    shape = dev[(synth.ROLE_Q, 0)].shape
    dk = {b: torch.zeros(shape, dtype=torch.float32, device="cuda") for b in range(n)}
    dv = {b: torch.zeros(shape, dtype=torch.float32, device="cuda") for b in range(n)}
    dq = {b: torch.zeros(shape, dtype=torch.float32, device="cuda") for b in range(n)}

    def source(j):
        a, b = zigzag_blocks(j, P)
        return (dev[(synth.ROLE_K, a)], dev[(synth.ROLE_K, b)], dev[(synth.ROLE_V, a)],
                dev[(synth.ROLE_V, b)], dk[a], dk[b], dv[a], dv[b])

    ring = ZigzagRing(shape, dev[(synth.ROLE_Q, 0)].dtype, backward=True)
    for rank in range(P):
        mine = zigzag_blocks(rank, P)
        qs = [dev[(synth.ROLE_Q, b)] for b in mine]
        dos = [dev[(synth.ROLE_DO, b)] for b in mine]
        states = [_lib.State(1, heads, sub.rows, d) for _ in range(2)]
        ring.run(states, qs, lambda j: source(j)[:4], rank, P, causal, sub.scale)
        outs = [_lib.finalize(st, torch.float32, ring.compute) for st in states]
        lses = [lse for _, lse in outs]
        deltas = [_lib.bwd_prepare(o, do, stream=ring.compute) for (o, _), do in zip(outs, dos)]
        ring.run_backward(qs, dos, lses, deltas, [dq[b] for b in mine], source, rank, P, causal,
                          sub.scale)
        torch.cuda.synchronize()
    cat = lambda role: np.concatenate([oracle_values(host[(role, b)], sub) for b in range(n)], axis=1)
    pos = np.arange(n * sub.rows)
    wq, wk, wv = backward.attention_backward(cat(synth.ROLE_Q), cat(synth.ROLE_K), cat(synth.ROLE_V),
                                             cat(synth.ROLE_DO), pos, pos, causal, sub.scale)
    rel = 2e-2 if dtype == "bf16" else 1e-4
    for b in range(n):
        sl = slice(b * sub.rows, (b + 1) * sub.rows)
        for got, want, name in ((dq[b], wq, "dQ"), (dk[b], wk, "dK"), (dv[b], wv, "dV")):
            g = got[0].cpu().numpy().astype(np.float64)
            w = want[:, sl]
            scale_ = max(float(np.max(np.abs(want))), 1e-30)
            err = float(np.max(np.abs(g - w)))
            assert np.isfinite(g).all() and err <= rel * scale_, (b, name, err, scale_)
        _say(f"  {sub.name} causal={causal} piece {b} ok")


@pytest.mark.parametrize("heads,d,rows,P,dtype", [(2, 128, 400, 3, "bf16"), (1, 64, 128, 4, "f32")])
@pytest.mark.parametrize("causal", [True, False])
def test_zigzag_fused_init_finalize_is_bit_identical(heads, d, rows, P, dtype, causal):
    """ZigzagRing.run with finalize_outs (each piece's init and finalize fused
    into its first and last product) gives exactly the separate-launch outputs."""
    wl = synth.Workload(f"zzf_{dtype}_h{heads}_d{d}_c{rows}_p{P}", 250 + rows + d, heads, d, rows,
                        P, dtype, causal, tuple(range(P)))
    sub = synth.zigzag_workload(wl)
    cache = gen_blocks(sub, [(r, b) for b in range(2 * P)
                             for r in (synth.ROLE_Q, synth.ROLE_K, synth.ROLE_V)])
    dev = {key: to_device(x, sub) for key, x in cache.items()}
    for rank in range(P):
        mine = zigzag_blocks(rank, P)
        qs = [dev[(synth.ROLE_Q, b)] for b in mine]

        def source(j):
            a, b = zigzag_blocks(j, P)
            return (dev[(synth.ROLE_K, a)], dev[(synth.ROLE_K, b)], dev[(synth.ROLE_V, a)],
                    dev[(synth.ROLE_V, b)])

        ring = ZigzagRing(qs[0].shape, qs[0].dtype)
        states = [_lib.State(1, heads, sub.rows, d) for _ in range(2)]
        ring.run(states, qs, source, rank, P, causal, sub.scale)
        want = [_lib.finalize(st, torch.float32, ring.compute) for st in states]
        for st in states:
            for t in (st.m, st.l, st.o):
                t.fill_(float("nan"))
        outs = [(torch.empty_like(w[0]), torch.empty_like(w[1])) for w in want]
        ring.run(states, qs, source, rank, P, causal, sub.scale, finalize_outs=outs)
        torch.cuda.synchronize()
        for (o, l), (wo, wlse) in zip(outs, want):
            assert torch.equal(o, wo) and torch.equal(l, wlse), (rank, causal)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rank", [7, 3, 0])
def test_bench_zigzag_path_every_row(rank):
    """The zigzag ring bench.py times (--partition zigzag) at the headline
    shape (32 heads, d = 128, 4096 tokens per rank in two pieces of 2048, 8
    ranks): each rank's two pieces in one block in position order, every
    visit one launch on row ranges of the blocks (ZigzagRing.run_block, split
    per piece where the fused init or finalize needs it), its own compute
    stream, the staging mode bench.py picks, timing events on every launch.
    Both pieces, every row and head, against the oracle."""
    import concurrent.futures as cf
    import contextlib
    from ring_attention_block_amd.hip_events import Event
    from ring_attention_block_amd.ring import launch_pairs, staging_for, zigzag_fused_launches
    wl = synth.WORKLOADS["causal_bf16_h32_d128_c4096_p8"]
    sub = synth.zigzag_workload(wl)
    P = wl.blocks
    mine = zigzag_blocks(rank, P)
    cache = gen_blocks(sub, [(synth.ROLE_Q, b) for b in mine] +
                       [(r, b) for b in range(2 * P) for r in (synth.ROLE_K, synth.ROLE_V)])
    dev = {key: to_device(x, sub) for key, x in cache.items()}
    q = torch.cat([dev[(synth.ROLE_Q, b)] for b in mine], dim=2)
    kv = {j: tuple(torch.cat([dev[(role, b)] for b in zigzag_blocks(j, P)], dim=2)
                   for role in (synth.ROLE_K, synth.ROLE_V)) for j in range(P)}
    plan = zigzag_fused_launches(rank, P, True)
    lightest = min(sum(launch_pairs(l, sub.rows) for l in ls) for _, ls in plan)
    staging = staging_for(wl.heads, lightest, 1, wl.head_dim, 0)
    compute = torch.cuda.Stream()
    st = _lib.State(1, wl.heads, 2 * sub.rows, wl.head_dim)
    out = (torch.full((1, wl.heads, 2 * sub.rows, wl.head_dim), float("nan"), device="cuda"),
           torch.full((1, wl.heads, 2 * sub.rows), float("nan"), device="cuda"))
    launched = sum(len(ls) for _, ls in plan)
    timers = []
    pool = iter([Event(timing=True) for _ in range(2 * launched)])
    ring = ZigzagRing((1, wl.heads, sub.rows, wl.head_dim), q.dtype, "cuda", compute_stream=compute,
                      staging=staging)
    _say(f"{sub.name} rank {rank}: staging {staging}, {launched} launches")
    ring.run_block(st, q, lambda j: kv[j], rank, P, True, sub.scale, step_timers=timers,
                   timer_events=pool, finalize_out=out)
    h = sub.rows
    outs = [(out[0][:, :, n * h:(n + 1) * h], out[1][:, :, n * h:(n + 1) * h]) for n in range(2)]
    torch.cuda.synchronize()
    assert len(timers) == launched

    try:
        from threadpoolctl import threadpool_limits
        one_blas_thread = threadpool_limits(limits=1)   # applies now, restores on exit
    except ImportError:       # pragma: no cover
        one_blas_thread = contextlib.nullcontext()
    want = {}
    with one_blas_thread, cf.ThreadPoolExecutor(max_workers=16) as ex:
        for piece in mine:
            def one(h, piece=piece):
                return oracle_rank(sub, piece, range(2 * P), True, head_sel=[h], cache=cache)
            parts = []
            for h0 in range(0, wl.heads, 8):
                parts += list(ex.map(one, range(h0, min(wl.heads, h0 + 8))))
                _say(f"  piece {piece}: oracle heads {h0}..{min(wl.heads, h0 + 8) - 1}")
            want[piece] = (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    to, tl = tol_for(sub)
    for piece, (o, lse) in zip(mine, outs):
        eo = assert_close(o[0].cpu().numpy(), want[piece][0], to, f"rank {rank} piece {piece} O")
        el = assert_close(lse[0].cpu().numpy(), want[piece][1], tl, f"rank {rank} piece {piece} LSE")
        _say(f"  piece {piece}, every row: max|dO|={eo:.2e} max|dLSE|={el:.2e}")
