"""GPU parity of the backward ring step (ra_bwd_prepare, ra_bwd_step and the
backward ring of RingEmulator) against the fp64 backward oracle.

"Ring Attention：把超长序列沿设备环流动", section "Backward 需要让梯度也沿环传播":
the query owner accumulates dQ, the dK and dV of a key/value block accumulate
while it travels the ring and return to its owner, and the probabilities are
recomputed from the saved log-sum-exp.  Inputs come from
ring_attention_block_amd.synth; expected values from oracle/ only.

Tolerance (max abs error relative to the largest reference magnitude of the
tensor): fp32 inputs 1e-4; bf16 inputs 2e-2, the bf16 kernels rounding the
probabilities and dS to bf16 (2^-9 relative per term) before their products,
as the forward rounds P.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import backward, dense
from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.ring import RingEmulator

from _helpers import gen_blocks, oracle_values, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.lib()


def _rel_tol(wl):
    return 2e-2 if wl.dtype == "bf16" else 1e-4


def _close(got, want, wl, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    scale = max(float(np.max(np.abs(want))), 1e-30)
    err = float(np.max(np.abs(got - want)))
    assert err <= _rel_tol(wl) * scale, f"{what}: max abs error {err:.3e} > {_rel_tol(wl):.0e} x {scale:.3e}"
    return err / scale


def _inputs(wl):
    jobs = [(r, j) for j in range(wl.blocks)
            for r in (synth.ROLE_Q, synth.ROLE_K, synth.ROLE_V, synth.ROLE_DO)]
    host = gen_blocks(wl, jobs)
    dev = {key: to_device(x, wl) for key, x in host.items()}
    f64 = {key: oracle_values(x, wl) for key, x in host.items()}
    return host, dev, f64


SMALL = [
    # (heads, head_dim, rows, blocks, dtype); bf16 runs the matrix-core
    # kernels, fp32 the general kernel.
    (2, 128, 200, 3, "bf16"),
    (1, 64, 130, 3, "f32"),
    (8, 128, 640, 2, "bf16"),
    (16, 128, 1000, 2, "bf16"),
    (4, 64, 300, 3, "bf16"),
    (8, 64, 1000, 2, "bf16"),
    (2, 64, 96, 2, "bf16"),
    (1, 128, 64, 2, "f32"),
    (1, 128, 1, 2, "bf16"),
    (1, 64, 7, 2, "bf16"),
]


@pytest.mark.parametrize("heads,d,rows,P,dtype", SMALL)
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_step_every_pair(heads, d, rows, P, dtype, causal):
    """Each (query block i, key block j) step against the oracle's per-block
    contribution, both fed the oracle's LSE and D."""
    wl = synth.Workload(f"bwd_{dtype}_h{heads}_d{d}_c{rows}_p{P}", 400 + rows + d, heads, d, rows,
                        P, dtype, causal, tuple(range(P)))
    _, dev, f64 = _inputs(wl)
    kall = np.concatenate([f64[(synth.ROLE_K, j)] for j in range(P)], axis=1)
    vall = np.concatenate([f64[(synth.ROLE_V, j)] for j in range(P)], axis=1)
    kpos = np.arange(P * rows)
    for i in range(P):
        qpos = dense.ring_positions(i, rows)
        q64, do64 = f64[(synth.ROLE_Q, i)], f64[(synth.ROLE_DO, i)]
        o, lse = dense.attention(q64, kall, vall, qpos, kpos, causal, wl.scale)
        delta = backward.row_dot(do64, o)
        lse_d = torch.tensor(lse[None], dtype=torch.float32, device="cuda").contiguous()
        del_d = torch.tensor(delta[None], dtype=torch.float32, device="cuda").contiguous()
        for j in range(P):
            shape = dev[(synth.ROLE_Q, i)].shape
            dq, dk, dv = (torch.zeros(shape, dtype=torch.float32, device="cuda") for _ in range(3))
            case = _lib.bwd_step(dev[(synth.ROLE_Q, i)], dev[(synth.ROLE_DO, i)], lse_d, del_d,
                                 dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)], dq, dk, dv,
                                 i, j, P, causal, wl.scale)
            torch.cuda.synchronize()
            wq, wk, wv = backward.block_backward(q64, f64[(synth.ROLE_K, j)], f64[(synth.ROLE_V, j)],
                                                 do64, lse, delta, qpos,
                                                 dense.ring_positions(j, rows), causal, wl.scale)
            if case == _lib.RA_CASE_SKIP:
                assert not dq.any() and not dk.any() and not dv.any()
                assert not wq.any() and not wk.any() and not wv.any()
                continue
            what = f"{wl.name} causal={causal} i={i} j={j}"
            e = [_close(dq[0].cpu().numpy(), wq, wl, what + " dQ"),
                 _close(dk[0].cpu().numpy(), wk, wl, what + " dK"),
                 _close(dv[0].cpu().numpy(), wv, wl, what + " dV")]
            _say(f"  {what}: rel err dQ {e[0]:.1e} dK {e[1]:.1e} dV {e[2]:.1e}")


@pytest.mark.parametrize("heads,d,rows,P,dtype", SMALL[:6])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_ring_gives_full_gradients(heads, d, rows, P, dtype, causal):
    """Every rank's forward ring, then every rank's backward ring (dK, dV of
    each block staged in, updated and sent on), against the dense gradients of
    the whole sequence."""
    wl = synth.Workload(f"bwdring_{dtype}_h{heads}_d{d}_c{rows}_p{P}", 500 + rows + d, heads, d,
                        rows, P, dtype, causal, tuple(range(P)))
    _, dev, f64 = _inputs(wl)
    shape = dev[(synth.ROLE_Q, 0)].shape
    kv = {j: (dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)]) for j in range(P)}
    dk = {j: torch.zeros(shape, dtype=torch.float32, device="cuda") for j in range(P)}
    dv = {j: torch.zeros(shape, dtype=torch.float32, device="cuda") for j in range(P)}
    fwd = RingEmulator(shape, dev[(synth.ROLE_Q, 0)].dtype)
    bwd = RingEmulator(shape, dev[(synth.ROLE_Q, 0)].dtype, compute_stream=fwd.compute,
                       extra_specs=[(shape, torch.float32), (shape, torch.float32)])
    dq = {}
    for i in range(P):
        st = _lib.State(*shape)
        fwd.run(st, dev[(synth.ROLE_Q, i)], lambda j: kv[j], i, P, causal, wl.scale)
        o, lse = _lib.finalize(st, torch.float32, fwd.compute)
        delta = _lib.bwd_prepare(o, dev[(synth.ROLE_DO, i)], stream=fwd.compute)
        dq[i] = torch.zeros(shape, dtype=torch.float32, device="cuda")
        bwd.run_backward(dev[(synth.ROLE_Q, i)], dev[(synth.ROLE_DO, i)], lse, delta, dq[i],
                         lambda j: (kv[j][0], kv[j][1], dk[j], dv[j]), i, P, causal, wl.scale)
    torch.cuda.synchronize()
    cat = lambda role: np.concatenate([f64[(role, j)] for j in range(P)], axis=1)
    pos = np.arange(P * rows)
    wq, wk, wv = backward.attention_backward(cat(synth.ROLE_Q), cat(synth.ROLE_K), cat(synth.ROLE_V),
                                             cat(synth.ROLE_DO), pos, pos, causal, wl.scale)
    for j in range(P):
        sl = slice(j * rows, (j + 1) * rows)
        what = f"{wl.name} causal={causal} block {j}"
        e = [_close(dq[j][0].cpu().numpy(), wq[:, sl], wl, what + " dQ"),
             _close(dk[j][0].cpu().numpy(), wk[:, sl], wl, what + " dK"),
             _close(dv[j][0].cpu().numpy(), wv[:, sl], wl, what + " dV")]
        _say(f"  {what}: rel err dQ {e[0]:.1e} dK {e[1]:.1e} dV {e[2]:.1e}")


@pytest.mark.parametrize("kv_block", [3, 7])
def test_bwd_step_headline_shape_sampled_heads(kv_block):
    """The step at the full size of the causal workload (32 heads, head_dim
    128, 4096 rows per block, query block 7 of 8) against the oracle on two
    whole heads.  LSE and D are those of attention over block kv_block alone
    (valid inputs of one step: P is then that block's softmax); the other
    heads get an upper bound of each row's scaled scores as LSE (P <= 1) and
    D = 0, so that every workgroup of the launch runs on finite data."""
    wl = synth.WORKLOADS["causal_bf16_h32_d128_c4096_p8"]
    i, j, heads = 7, kv_block, (5, 30)
    host = gen_blocks(wl, [(synth.ROLE_Q, i), (synth.ROLE_DO, i), (synth.ROLE_K, j), (synth.ROLE_V, j)])
    dev = {key: to_device(x, wl) for key, x in host.items()}
    f64 = {key: oracle_values(x, wl) for key, x in host.items()}
    q, do = f64[(synth.ROLE_Q, i)], f64[(synth.ROLE_DO, i)]
    k, v = f64[(synth.ROLE_K, j)], f64[(synth.ROLE_V, j)]
    qn = np.linalg.norm(q, axis=2)
    kmax = np.linalg.norm(k, axis=2).max(axis=1)
    lse = (wl.scale * qn * kmax[:, None]).astype(np.float32)
    delta = np.zeros_like(lse)
    qpos, kpos = dense.ring_positions(i, wl.rows), dense.ring_positions(j, wl.rows)
    causal = True
    want = {}
    for hd in heads:
        o, l = dense.attention(q[hd:hd + 1], k[hd:hd + 1], v[hd:hd + 1], qpos, kpos, causal, wl.scale)
        dl = backward.row_dot(do[hd:hd + 1], o)
        lse[hd], delta[hd] = l[0], dl[0]
        want[hd] = backward.block_backward(q[hd:hd + 1], k[hd:hd + 1], v[hd:hd + 1], do[hd:hd + 1],
                                           l, dl, qpos, kpos, causal, wl.scale)
    shape = dev[(synth.ROLE_Q, i)].shape
    dq, dk, dv = (torch.zeros(shape, dtype=torch.float32, device="cuda") for _ in range(3))
    lse_d = torch.from_numpy(lse[None]).cuda()
    del_d = torch.from_numpy(delta[None]).cuda()
    _say(f"  bwd_step headline shape i={i} j={j}")
    _lib.bwd_step(dev[(synth.ROLE_Q, i)], dev[(synth.ROLE_DO, i)], lse_d, del_d,
                  dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)], dq, dk, dv, i, j, wl.blocks, causal,
                  wl.scale)
    torch.cuda.synchronize()
    for t, name in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert torch.isfinite(t).all(), f"{name}: non-finite values"
    for hd in heads:
        wq, wk, wv = want[hd]
        e = [_close(dq[0, hd].cpu().numpy(), wq[0], wl, f"head {hd} dQ"),
             _close(dk[0, hd].cpu().numpy(), wk[0], wl, f"head {hd} dK"),
             _close(dv[0, hd].cpu().numpy(), wv[0], wl, f"head {hd} dV")]
        _say(f"  j={j} head {hd}: rel err dQ {e[0]:.1e} dK {e[1]:.1e} dV {e[2]:.1e}")


@pytest.mark.parametrize("heads,d,rows,o_dtype,do_dtype", [
    (3, 128, 37, "f32", "bf16"), (2, 64, 100, "bf16", "bf16"), (1, 128, 1, "f32", "f32"),
    (32, 128, 4096, "f32", "bf16")])
def test_bwd_prepare_row_dot(heads, d, rows, o_dtype, do_dtype):
    """ra_bwd_prepare against the oracle's D = rowsum(dO * O) (fp32 sums of
    products of exactly representable inputs: relative error ~ d * 2^-24)."""
    wl_o = synth.Workload("prep_o", 71 + rows, heads, d, rows, 1, o_dtype, False, (0,))
    wl_d = synth.Workload("prep_do", 72 + rows, heads, d, rows, 1, do_dtype, False, (0,))
    o_h = synth.block(wl_o, synth.ROLE_Q, 0)
    d_h = synth.block(wl_d, synth.ROLE_DO, 0)
    dq = torch.full((1, heads, rows, d), float("nan"), device="cuda")
    got = _lib.bwd_prepare(to_device(o_h, wl_o), to_device(d_h, wl_d), dq=dq)
    torch.cuda.synchronize()
    assert bool((dq == 0).all())                 # the dQ accumulator is cleared in the same launch
    want = backward.row_dot(oracle_values(d_h, wl_d), oracle_values(o_h, wl_o))
    bound = np.sum(np.abs(oracle_values(d_h, wl_d) * oracle_values(o_h, wl_o)), axis=-1)
    err = np.abs(got[0].cpu().numpy().astype(np.float64) - want)
    assert np.all(err <= 1e-6 * d * bound + 1e-30), float(np.max(err / (bound + 1e-30)))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kv_block", [30, 31])
def test_bwd_step_longshare_shape_sampled(kv_block):
    """The step at the full size of the head_dim-64 workload (16 heads, 16384
    rows per block, query block 31 of 32) against the oracle on sampled query
    rows (dQ) and sampled keys (dK, dV) of two heads.  Those heads get the LSE
    and D of attention over block kv_block alone, computed by the oracle; the
    other heads an upper bound of each row's scaled scores as LSE and D = 0."""
    wl = synth.WORKLOADS["longshare_bf16_h16_d64_c16384_p32"]
    i, j, heads = 31, kv_block, (3, 12)
    host = gen_blocks(wl, [(synth.ROLE_Q, i), (synth.ROLE_DO, i), (synth.ROLE_K, j), (synth.ROLE_V, j)])
    dev = {key: to_device(x, wl) for key, x in host.items()}
    f64 = {key: oracle_values(x, wl) for key, x in host.items()}
    q, do = f64[(synth.ROLE_Q, i)], f64[(synth.ROLE_DO, i)]
    k, v = f64[(synth.ROLE_K, j)], f64[(synth.ROLE_V, j)]
    lse = (wl.scale * np.linalg.norm(q, axis=2) * np.linalg.norm(k, axis=2).max(axis=1)[:, None])
    lse = lse.astype(np.float32)
    delta = np.zeros_like(lse)
    qpos, kpos = dense.ring_positions(i, wl.rows), dense.ring_positions(j, wl.rows)
    for hd in heads:
        o, l = dense.attention(q[hd:hd + 1], k[hd:hd + 1], v[hd:hd + 1], qpos, kpos, True, wl.scale)
        lse[hd], delta[hd] = l[0], backward.row_dot(do[hd:hd + 1], o)[0]
    shape = dev[(synth.ROLE_Q, i)].shape
    dq, dk, dv = (torch.zeros(shape, dtype=torch.float32, device="cuda") for _ in range(3))
    _say(f"  bwd_step d64 shape i={i} j={j}")
    _lib.bwd_step(dev[(synth.ROLE_Q, i)], dev[(synth.ROLE_DO, i)], torch.from_numpy(lse[None]).cuda(),
                  torch.from_numpy(delta[None]).cuda(), dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)],
                  dq, dk, dv, i, j, wl.blocks, True, wl.scale)
    torch.cuda.synchronize()
    for t, name in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert torch.isfinite(t).all(), f"{name}: non-finite values"
    rows = synth.sample_rows(wl.seed, wl.rows, 96)
    for hd in heads:
        hs = slice(hd, hd + 1)
        l64, d64 = lse[hs].astype(np.float64), delta[hs].astype(np.float64)
        # dQ of the sampled rows: those rows against every key of the block.
        wq, _, _ = backward.block_backward(q[hs][:, rows], k[hs], v[hs], do[hs][:, rows], l64[:, rows],
                                           d64[:, rows], qpos[rows], kpos, True, wl.scale)
        # dK, dV of the sampled keys: every query row against those keys.
        _, wk, wv = backward.block_backward(q[hs], k[hs][:, rows], v[hs][:, rows], do[hs], l64, d64,
                                            qpos, kpos[rows], True, wl.scale)
        e = [_close(dq[0, hd, rows].cpu().numpy(), wq[0], wl, f"head {hd} dQ"),
             _close(dk[0, hd, rows].cpu().numpy(), wk[0], wl, f"head {hd} dK"),
             _close(dv[0, hd, rows].cpu().numpy(), wv[0], wl, f"head {hd} dV")]
        _say(f"  j={j} head {hd}: rel err dQ {e[0]:.1e} dK {e[1]:.1e} dV {e[2]:.1e}")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (64, "f32")])
def test_bwd_batch_is_an_outer_head_axis(d, dtype):
    """ra_bwd_step with batch 2 on [2, H, rows, d] = the batch-1 call on 2H
    heads, bit-identically for the matrix-core path (no atomics) and within
    the tolerance for the general kernel (fp32 atomics)."""
    heads, rows, P = 2, 200, 2
    wl = synth.Workload(f"bwdbatch_{dtype}_d{d}", 800 + d, 2 * heads, d, rows, P, dtype, True, (1,))
    _, dev, f64 = _inputs(wl)
    o, lse = dense.attention(f64[(synth.ROLE_Q, 1)], np.concatenate([f64[(synth.ROLE_K, j)] for j in range(P)], 1),
                             np.concatenate([f64[(synth.ROLE_V, j)] for j in range(P)], 1),
                             dense.ring_positions(1, rows), np.arange(P * rows), True, wl.scale)
    delta = backward.row_dot(f64[(synth.ROLE_DO, 1)], o)
    out = []
    for batch in (1, 2):
        shape = (batch, 2 * heads // batch, rows, d)
        v = lambda t: t.view(shape)
        lse_d = torch.tensor(lse, dtype=torch.float32, device="cuda").view(shape[:3])
        del_d = torch.tensor(delta, dtype=torch.float32, device="cuda").view(shape[:3])
        g = [torch.zeros(shape, dtype=torch.float32, device="cuda") for _ in range(3)]
        for j in range(P):
            _lib.bwd_step(v(dev[(synth.ROLE_Q, 1)]), v(dev[(synth.ROLE_DO, 1)]), lse_d, del_d,
                          v(dev[(synth.ROLE_K, j)]), v(dev[(synth.ROLE_V, j)]), g[0], g[1], g[2], 1, j, P,
                          True, wl.scale)
        torch.cuda.synchronize()
        out.append([t.reshape(1, 2 * heads, rows, d) for t in g])
    for a, b, name in zip(out[0], out[1], ("dQ", "dK", "dV")):
        if dtype == "bf16":
            assert torch.equal(a, b), name
        else:
            assert float((a - b).abs().max()) <= 1e-5 * float(a.abs().max()), name


@pytest.mark.timeout(1200)
def test_bench_backward_path_every_head():
    """The backward ring bench.py times (--backward): rank 7 of the causal
    workload (32 heads, head_dim 128, 4096 rows per block, 8 blocks) on its
    own compute stream: forward ring, finalize, ra_bwd_prepare (which also
    zeroes dQ), then the backward ring with dK, dV travelling with the blocks
    and timing events bound to every step (ra_bwd_step_timed).  dQ of the
    rank and the rank's contribution to dK, dV of every block, on every head
    and row, against the oracle (forward over the 8 visible blocks, D from its
    output, then each block's backward from the oracle's LSE)."""
    import concurrent.futures as cf
    import contextlib
    from ring_attention_block_amd.hip_events import Event
    wl = synth.WORKLOADS["causal_bf16_h32_d128_c4096_p8"]
    i, P, causal = 7, wl.blocks, True
    jobs = [(synth.ROLE_Q, i), (synth.ROLE_DO, i)] + [(r, j) for j in range(P)
                                                      for r in (synth.ROLE_K, synth.ROLE_V)]
    host = gen_blocks(wl, jobs)
    dev = {key: to_device(x, wl) for key, x in host.items()}
    q, do = dev[(synth.ROLE_Q, i)], dev[(synth.ROLE_DO, i)]
    kv = {j: (dev[(synth.ROLE_K, j)], dev[(synth.ROLE_V, j)]) for j in range(P)}
    shape = tuple(q.shape)
    compute = torch.cuda.Stream()
    f32 = torch.float32
    ring = RingEmulator(shape, q.dtype, "cuda", compute_stream=compute,
                        extra_specs=[(shape, f32), (shape, f32)])
    st = _lib.State(*shape)
    ring.run(st, q, lambda j: kv[j], i, P, causal, wl.scale)
    o, lse = _lib.finalize(st, f32, compute)
    grads = {j: (torch.zeros(shape, dtype=f32, device="cuda"), torch.zeros(shape, dtype=f32, device="cuda"))
             for j in range(P)}
    dq = torch.full(shape, float("nan"), dtype=f32, device="cuda")   # ra_bwd_prepare zeroes it
    delta = torch.empty(shape[:3], dtype=f32, device="cuda")
    _lib.bwd_prepare(o, do, delta, stream=compute, dq=dq)
    timers = []
    pool = iter([Event(timing=True) for _ in range(2 * P)])
    _say(f"  {wl.name} rank {i}: backward ring as bench.py runs it")
    ring.run_backward(q, do, lse, delta, dq, lambda j: (kv[j][0], kv[j][1], grads[j][0], grads[j][1]),
                      i, P, causal, wl.scale, step_timers=timers, timer_events=pool)
    torch.cuda.synchronize()
    assert len(timers) == P and all(a.elapsed_time(b) > 0 for _, a, b in timers)
    got_dq = dq[0].cpu().numpy()
    got_dk = {j: grads[j][0][0].cpu().numpy() for j in range(P)}
    got_dv = {j: grads[j][1][0].cpu().numpy() for j in range(P)}
    for t in [got_dq] + list(got_dk.values()) + list(got_dv.values()):
        assert np.isfinite(t).all()

    qf, dof = oracle_values(host[(synth.ROLE_Q, i)], wl), oracle_values(host[(synth.ROLE_DO, i)], wl)
    kf = {j: oracle_values(host[(synth.ROLE_K, j)], wl) for j in range(P)}
    vf = {j: oracle_values(host[(synth.ROLE_V, j)], wl) for j in range(P)}
    qpos = dense.ring_positions(i, wl.rows)

    def one_head(hd):
        sl = slice(hd, hd + 1)
        kall = np.concatenate([kf[j][sl] for j in range(P)], axis=1)
        vall = np.concatenate([vf[j][sl] for j in range(P)], axis=1)
        kpos_all = np.concatenate([dense.ring_positions(j, wl.rows) for j in range(P)])
        o_h, lse_h = dense.attention(qf[sl], kall, vall, qpos, kpos_all, causal, wl.scale)
        d_h = backward.row_dot(dof[sl], o_h)
        wq = np.zeros_like(qf[sl])
        wk, wv = {}, {}
        for j in range(P):
            bq, wk[j], wv[j] = backward.block_backward(qf[sl], kf[j][sl], vf[j][sl], dof[sl], lse_h, d_h,
                                                       qpos, dense.ring_positions(j, wl.rows), causal,
                                                       wl.scale)
            wq = wq + bq
        return wq[0], {j: wk[j][0] for j in wk}, {j: wv[j][0] for j in wv}

    try:
        from threadpoolctl import threadpool_limits
        one_blas_thread = threadpool_limits(limits=1)
    except ImportError:       # pragma: no cover
        one_blas_thread = contextlib.nullcontext()
    _say(f"  oracle backward over {wl.heads} heads")
    with one_blas_thread, cf.ThreadPoolExecutor(max_workers=16) as ex:
        want = list(ex.map(one_head, range(wl.heads)))
    wq = np.stack([w[0] for w in want])
    e = [_close(got_dq, wq, wl, "rank 7 dQ")]
    for j in range(P):
        e.append(_close(got_dk[j], np.stack([w[1][j] for w in want]), wl, f"block {j} dK"))
        e.append(_close(got_dv[j], np.stack([w[2][j] for w in want]), wl, f"block {j} dV"))
    _say(f"  every head and row: max rel err {max(e):.1e} (dQ {e[0]:.1e})")
