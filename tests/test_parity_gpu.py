"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Every input comes from ring_attention_block_amd.synth; every expected value
from oracle/.  Tolerances are max abs error: fp32 inputs 1e-5 (O) and 1e-5
(LSE); bf16 inputs with fp32 accumulation 2e-2 (O) and 5e-3 (LSE).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.ring import RingEmulator, ring_order

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
    """Seeded blocks of one workload, resident on the device; the host copies
    are kept in `cache` for the oracle."""

    def __init__(self, wl, rank, blocks=None):
        self.wl = wl
        blocks = list(range(wl.blocks) if blocks is None else blocks)
        jobs = [(synth.ROLE_Q, rank)] + [(r, j) for j in blocks
                                         for r in (synth.ROLE_K, synth.ROLE_V)]
        self.cache = gen_blocks(wl, jobs)
        self.q = to_device(self.cache[(synth.ROLE_Q, rank)], wl)
        self.kv = {j: (to_device(self.cache[(synth.ROLE_K, j)], wl),
                       to_device(self.cache[(synth.ROLE_V, j)], wl)) for j in blocks}

    def set_rank(self, rank):
        key = (synth.ROLE_Q, rank)
        if key not in self.cache:
            self.cache[key] = synth.block(self.wl, *key)
        self.q = to_device(self.cache[key], self.wl)


def run_ring(inp, rank, causal, order=None, out_dtype=torch.float32):
    wl = inp.wl
    st = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
    emu = RingEmulator(inp.q.shape, inp.q.dtype)
    cases = emu.run(st, inp.q, lambda j: inp.kv[j], rank, wl.blocks, causal, wl.scale,
                    order=order)
    o, lse = _lib.finalize(st, out_dtype, emu.compute)
    torch.cuda.synchronize()
    return st, o, lse, cases


def _check(wl, o, lse, rank, causal, blocks=None, rows=None, cache=None, what=""):
    blocks = list(range(wl.blocks)) if blocks is None else blocks
    want_o, want_lse = oracle_rank(wl, rank, blocks, causal, row_sel=rows, cache=cache)
    got_o = o[0].float().cpu().numpy()
    got_lse = lse[0].cpu().numpy()
    if rows is not None:
        got_o, got_lse = got_o[:, rows], got_lse[:, rows]
    to, tl = tol_for(wl)
    eo = assert_close(got_o, want_o, to, f"{what} O")
    el = assert_close(got_lse, want_lse, tl, f"{what} LSE")
    _say(f"  {what}: max|dO|={eo:.2e} max|dLSE|={el:.2e}")


# --------------------------------------------------------------- small / ragged

TINY = synth.WORKLOADS["tiny_f32_h1_d64_c128_p4"]


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_f32_every_rank(causal):
    for rank in range(TINY.blocks):
        _say(f"tiny f32 causal={causal} rank={rank}")
        inp = Inputs(TINY, rank)
        _, o, lse, cases = run_ring(inp, rank, causal)
        _check(TINY, o, lse, rank, causal, cache=inp.cache, what=f"rank {rank}")


SMALL = [
    # (heads, head_dim, rows, blocks, dtype): several tiles and a ragged tail
    (2, 128, 200, 3, "bf16"),
    (3, 64, 300, 3, "bf16"),
    (1, 128, 1, 4, "bf16"),
    (2, 64, 129, 2, "bf16"),
    (1, 128, 64, 2, "bf16"),
    (2, 128, 333, 2, "f32"),
    (1, 64, 70, 3, "f32"),
    # long enough that masked launches run whole tiles before their masked ones
    (2, 128, 1000, 2, "bf16"),
    (2, 128, 512, 2, "bf16"),
    (1, 64, 777, 2, "bf16"),
]


@pytest.mark.parametrize("heads,d,rows,P,dtype", SMALL)
@pytest.mark.parametrize("causal", [False, True])
def test_small_ragged_every_rank(heads, d, rows, P, dtype, causal):
    wl = synth.Workload(f"small_{dtype}_h{heads}_d{d}_c{rows}_p{P}", 100 + rows + d, heads, d,
                        rows, P, dtype, causal, tuple(range(P)))
    for rank in range(P):
        _say(f"{wl.name} causal={causal} rank={rank}")
        inp = Inputs(wl, rank)
        _, o, lse, _ = run_ring(inp, rank, causal)
        _check(wl, o, lse, rank, causal, cache=inp.cache, what=f"rank {rank}")


def test_bf16_output_and_finalize_keeps_state():
    wl = synth.Workload("small_bf16_out", 7, 2, 128, 256, 2, "bf16", True, (1,))
    inp = Inputs(wl, 1)
    st, o32, lse, _ = run_ring(inp, 1, True)
    m0, l0, O0 = st.m.clone(), st.l.clone(), st.o.clone()
    o16, lse2 = _lib.finalize(st, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(m0, st.m) and torch.equal(l0, st.l) and torch.equal(O0, st.o)
    assert torch.equal(lse, lse2)
    assert torch.equal(o16, o32.to(torch.bfloat16))   # same round-to-nearest-even
    _check(wl, o16, lse2, 1, True, cache=inp.cache, what="bf16 out")


def test_skip_step_leaves_state_bit_identical():
    wl = synth.Workload("small_skip", 8, 2, 128, 192, 4, "bf16", True, (1,))
    inp = Inputs(wl, 1)
    st, _, _, _ = run_ring(inp, 1, True)
    before = (st.m.clone(), st.l.clone(), st.o.clone())
    for j in (2, 3):
        assert _lib.step(st, inp.q, *inp.kv[j], 1, j, 4, True, wl.scale) == _lib.RA_CASE_SKIP
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, (st.m, st.l, st.o)))


def test_staged_ring_is_bit_identical_to_direct_calls():
    """Side-stream staging and buffer swaps must not change a single bit: the
    same steps called directly on the resident blocks give the same state."""
    wl = synth.Workload("small_hazard", 9, 4, 128, 1024, 6, "bf16", True, (5,))
    inp = Inputs(wl, 5)
    st_ring, _, _, _ = run_ring(inp, 5, True)
    st = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
    _lib.state_init(st)
    for j in ring_order(5, wl.blocks):
        _lib.step(st, inp.q, *inp.kv[j], 5, j, wl.blocks, True, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(st.m, st_ring.m) and torch.equal(st.l, st_ring.l)
    assert torch.equal(st.o, st_ring.o)


def test_merge_identity_and_partition():
    wl = synth.Workload("small_merge", 10, 2, 64, 320, 4, "bf16", True, (3,))
    inp = Inputs(wl, 3)
    halves = [[3, 1], [2, 0]]
    states = []
    for part in halves:
        st = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
        _lib.state_init(st)
        for j in part:
            _lib.step(st, inp.q, *inp.kv[j], 3, j, wl.blocks, True, wl.scale)
        states.append(st)
    empty = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
    _lib.state_init(empty)
    keep = (states[0].m.clone(), states[0].l.clone(), states[0].o.clone())
    _lib.lse_merge(states[0], empty)                       # x (+) empty = x, bit-exact
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(keep, (states[0].m, states[0].l, states[0].o)))
    e2 = _lib.State(1, wl.heads, wl.rows, wl.head_dim)
    _lib.state_init(e2)
    _lib.lse_merge(e2, states[1])                          # empty (+) y = y, bit-exact
    torch.cuda.synchronize()
    assert torch.equal(e2.m, states[1].m) and torch.equal(e2.l, states[1].l)
    assert torch.equal(e2.o, states[1].o)
    _lib.lse_merge(states[0], states[1])
    o, lse = _lib.finalize(states[0])
    torch.cuda.synchronize()
    _check(wl, o, lse, 3, True, cache=inp.cache, what="merged halves")


# --------------------------------------------------------------- full sizes

def _rows_sample(wl, count):
    return synth.sample_rows(wl.seed, wl.rows, count)


C2 = synth.WORKLOADS["causal_bf16_h32_d128_c4096_p8"]


@pytest.mark.timeout(900)
def test_causal_bf16_h32_d128_c4096_ranks():
    inp = Inputs(C2, 0)
    for rank in C2.ranks:
        _say(f"{C2.name} rank={rank}")
        inp.set_rank(rank)
        _, o, lse, cases = run_ring(inp, rank, True)
        assert cases.count(_lib.RA_CASE_DIAG) == 1
        assert cases.count(_lib.RA_CASE_FULL) == rank
        rows = _rows_sample(C2, 64)
        _check(C2, o, lse, rank, True, blocks=list(range(rank + 1)), rows=rows,
               cache=inp.cache, what=f"rank {rank}, {len(rows)} rows x {C2.heads} heads")


C3 = synth.WORKLOADS["rescale_bf16_h8_d128_c2048_p16"]


@pytest.mark.timeout(900)
def test_rescale_stress_forward_and_reversed():
    rank = 15
    inp = Inputs(C3, rank)
    fwd = ring_order(rank, C3.blocks)
    rows = _rows_sample(C3, 256)
    cache = inp.cache
    res = {}
    for name, order in (("ring order", fwd), ("reversed", fwd[::-1])):
        _say(f"{C3.name} {name}")
        st, o, lse, _ = run_ring(inp, rank, False, order=order)
        res[name] = (o, lse)
        _check(C3, o, lse, rank, False, rows=rows, cache=cache, what=name)
    # the two orders agree with each other on every row
    (o1, l1), (o2, l2) = res.values()
    assert float((o1 - o2).abs().max()) <= 2e-2
    assert float((l1 - l2).abs().max()) <= 5e-3


C4 = synth.WORKLOADS["longshare_bf16_h16_d64_c16384_p32"]


@pytest.mark.timeout(1200)
def test_longshare_d64_half_rings_merged():
    rank = 31
    inp = Inputs(C4, rank)
    order = ring_order(rank, C4.blocks)
    rows = _rows_sample(C4, 256)
    cache = inp.cache
    emu = RingEmulator(inp.q.shape, inp.q.dtype)
    states = []
    for half in (order[:16], order[16:]):
        st = _lib.State(1, C4.heads, C4.rows, C4.head_dim)
        emu.run(st, inp.q, lambda j: inp.kv[j], rank, C4.blocks, True, C4.scale, order=half)
        states.append(st)
    for st, half, name in zip(states, (order[:16], order[16:]), ("half A", "half B")):
        o, lse = _lib.finalize(st)
        torch.cuda.synchronize()
        _say(f"{C4.name} {name}")
        _check(C4, o, lse, rank, True, blocks=sorted(half), rows=rows, cache=cache, what=name)
    _lib.lse_merge(states[0], states[1], emu.compute)
    o, lse = _lib.finalize(states[0], stream=emu.compute)
    torch.cuda.synchronize()
    _check(C4, o, lse, rank, True, rows=rows, cache=cache, what="merged")


C5 = synth.WORKLOADS["million_bf16_h8_d128_c16384_p64"]


@pytest.mark.timeout(1200)
def test_million_token_rank_sampled_rows():
    rank = 63
    _say(f"{C5.name}: generating {C5.blocks} blocks")
    inp = Inputs(C5, rank)
    _, o, lse, cases = run_ring(inp, rank, True)
    assert cases.count(_lib.RA_CASE_FULL) == 63 and cases.count(_lib.RA_CASE_DIAG) == 1
    rows = _rows_sample(C5, 256)
    _check(C5, o, lse, rank, True, rows=rows, cache=inp.cache,
           what=f"{len(rows)} rows x {C5.heads} heads")


@pytest.mark.parametrize("d,rows,dtype", [(128, 300, "bf16"), (64, 200, "bf16"), (128, 130, "f32")])
def test_batch_is_an_outer_head_axis(d, rows, dtype):
    """[B, H, rows, d] with B = 2 is laid out as [1, 2H, rows, d]: a batch-2 ring
    step must give bit-identical state to the batch-1 call on 2H heads, and
    both match the oracle."""
    heads, P, rank = 3, 3, 2
    wl = synth.Workload(f"batch_{dtype}_d{d}_c{rows}", 700 + rows + d, 2 * heads, d, rows, P, dtype,
                        True, (rank,))
    inp = Inputs(wl, rank)
    results = []
    for batch in (1, 2):
        shape = (batch, 2 * heads // batch, rows, d)
        st = _lib.State(*shape)
        emu = RingEmulator(shape, inp.q.dtype)
        view = lambda t: t.view(shape)
        emu.run(st, view(inp.q), lambda j: (view(inp.kv[j][0]), view(inp.kv[j][1])), rank, P, True,
                wl.scale)
        o, lse = _lib.finalize(st, torch.float32, emu.compute)
        torch.cuda.synchronize()
        results.append((o.reshape(1, 2 * heads, rows, d), lse.reshape(1, 2 * heads, rows)))
    assert torch.equal(results[0][0], results[1][0]) and torch.equal(results[0][1], results[1][1])
    _check(wl, results[1][0], results[1][1], rank, True, cache=inp.cache, what=f"batch 2 {wl.name}")


FUSED = [(2, 128, 300, 3, "bf16"), (1, 64, 200, 4, "f32"), (3, 64, 129, 2, "bf16")]


@pytest.mark.parametrize("heads,d,rows,P,dtype", FUSED)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fused_init_finalize_ring_is_bit_identical(heads, d, rows, P, dtype, causal, out_dtype):
    """ra_step_ex: the ring with init fused into its first step (state not read:
    it is filled with NaN first) and finalize into its last gives exactly the
    outputs of the ring with separate ra_state_init and ra_finalize."""
    wl = synth.Workload(f"fused_{dtype}_h{heads}_d{d}_c{rows}_p{P}", 900 + rows + d, heads, d, rows,
                        P, dtype, causal, tuple(range(P)))
    inp = Inputs(wl, 0)
    for rank in range(P):
        inp.set_rank(rank)
        st = _lib.State(1, heads, rows, d)
        emu = RingEmulator(inp.q.shape, inp.q.dtype)
        emu.run(st, inp.q, lambda j: inp.kv[j], rank, P, causal, wl.scale)
        want = _lib.finalize(st, out_dtype, emu.compute)
        for t in (st.m, st.l, st.o):
            t.fill_(float("nan"))
        o = torch.empty(want[0].shape, dtype=out_dtype, device="cuda")
        lse = torch.empty(want[1].shape, dtype=torch.float32, device="cuda")
        emu.run(st, inp.q, lambda j: inp.kv[j], rank, P, causal, wl.scale, finalize_out=(o, lse))
        torch.cuda.synchronize()
        assert torch.equal(o, want[0]) and torch.equal(lse, want[1]), (rank, causal)
        if out_dtype == torch.float32:
            _check(wl, o, lse, rank, causal, cache=inp.cache, what=f"fused {wl.name} rank {rank}")


def test_step_ex_finalize_leaves_state_and_skip_applies_flags():
    wl = synth.Workload("stepex_bf16", 950, 2, 128, 192, 2, "bf16", True, (0, 1))
    inp = Inputs(wl, 1)
    st = _lib.State(1, 2, 192, 128)
    _lib.state_init(st)
    _lib.step(st, inp.q, *inp.kv[1], 1, 1, 2, True, wl.scale)
    before = [t.clone() for t in (st.m, st.l, st.o)]
    o = torch.empty(st.o.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(st.m.shape, dtype=torch.float32, device="cuda")
    _lib.step(st, inp.q, *inp.kv[0], 1, 0, 2, True, wl.scale, flags=_lib.RA_STEP_FINALIZE,
              o_out=o, lse_out=lse)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, (st.m, st.l, st.o)))
    _check(wl, o, lse, 1, True, cache=inp.cache, what="finalizing step")
    # A skipped block still applies both flags: empty state, O = 0, LSE = -inf.
    case = _lib.step(st, inp.q, *inp.kv[1], 0, 1, 2, True, wl.scale,
                     flags=_lib.RA_STEP_FRESH | _lib.RA_STEP_FINALIZE, o_out=o, lse_out=lse)
    torch.cuda.synchronize()
    assert case == _lib.RA_CASE_SKIP
    assert not o.any() and bool(torch.isneginf(lse).all()) and bool(torch.isneginf(st.m).all())
