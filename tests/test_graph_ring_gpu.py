"""GPU: a ring captured once as a HIP graph and replayed (what bench.py does
for its untimed rings) gives the eager ring's results bit for bit, on every
replay, with eager rings, other work and synchronisations between replays;
with the staging on a side stream and with the staging carried by the step
launches."""
import sys

import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.hip_events import Event
from ring_attention_block_amd.ring import RingEmulator, ZigzagRing, key_split_for, ring_order, split_keys, zigzag_blocks

from _helpers import gen_blocks, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.lib()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _replays_match(one_ring, copy_stream, compute, outs):
    """copy_stream None: the ring runs on the compute stream alone (staging
    carried by the step launches)."""
    join = Event()

    def joined():
        one_ring()
        if copy_stream is not None:
            join.record(copy_stream)
            join.wait(compute)

    joined()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        joined()
    torch.cuda.synchronize()
    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(compute):
            g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), f"replay {i} differs from the eager ring"
        joined()   # eager ring between replays
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), f"eager ring after replay {i} differs"


# (name, dtype, heads, d, rows, P, rank, causal)
CASES = [
    ("causal_rank3", "bf16", 4, 128, 512, 4, 3, True),
    ("causal_rank0_skips", "bf16", 2, 64, 300, 4, 0, True),
    ("noncausal_key_split", "bf16", 8, 128, 512, 3, 2, False),
    ("f32_causal", "f32", 2, 64, 200, 3, 2, True),
]


@pytest.mark.parametrize("staging", ["side", "fused"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_captured_ring_replays_bit_identically(case, staging):
    name, dtype, heads, d, rows, P, rank, causal = case
    wl = synth.Workload(f"graph_{name}", 70 + rows, heads, d, rows, P, dtype, causal, (rank,))
    jobs = [(synth.ROLE_Q, rank)] + [(r, j) for j in range(P) for r in (synth.ROLE_K, synth.ROLE_V)]
    host = gen_blocks(wl, jobs)
    q = to_device(host[(synth.ROLE_Q, rank)], wl)
    kv = {j: (to_device(host[(synth.ROLE_K, j)], wl), to_device(host[(synth.ROLE_V, j)], wl)) for j in range(P)}
    ks = key_split_for(heads, rows, rows, causal)
    if ks > 1:
        kv = {j: (split_keys(k, ks), split_keys(v, ks)) for j, (k, v) in kv.items()}
    _say(f"{name}: key split {ks}, {staging} staging")
    compute = torch.cuda.Stream()
    st = _lib.State(ks, heads, rows, d)
    emu = RingEmulator(kv[0][0].shape, q.dtype, compute_stream=compute, staging=staging)
    o = torch.empty((1, heads, rows, d), device="cuda")
    lse = torch.empty((1, heads, rows), device="cuda")
    _replays_match(lambda: emu.run(st, q, lambda j: kv[j], rank, P, causal, wl.scale,
                                   finalize_out=(o, lse), key_split=ks),
                   emu.copy if staging == "side" else None, compute, [o, lse])


@pytest.mark.parametrize("staging", ["side", "fused"])
def test_captured_zigzag_ring_replays_bit_identically(staging):
    heads, d, rows, P, rank = 2, 128, 256, 4, 1
    wl = synth.Workload("graph_zigzag", 91, heads, d, rows, P, "bf16", True, (rank,))
    zw = synth.zigzag_workload(wl)
    mine = zigzag_blocks(rank, P)
    jobs = [(synth.ROLE_Q, b) for b in mine] + [(r, b) for b in range(zw.blocks) for r in (synth.ROLE_K, synth.ROLE_V)]
    host = gen_blocks(zw, jobs)
    qs = [to_device(host[(synth.ROLE_Q, b)], zw) for b in mine]
    kv = {b: (to_device(host[(synth.ROLE_K, b)], zw), to_device(host[(synth.ROLE_V, b)], zw)) for b in range(zw.blocks)}

    def source(j):
        a, b = zigzag_blocks(j, P)
        return kv[a][0], kv[b][0], kv[a][1], kv[b][1]

    compute = torch.cuda.Stream()
    states = [_lib.State(1, heads, zw.rows, d) for _ in range(2)]
    zz = ZigzagRing(qs[0].shape, qs[0].dtype, compute_stream=compute, staging=staging)
    outs = [(torch.empty(st.o.shape, device="cuda"), torch.empty(st.m.shape, device="cuda")) for st in states]
    _replays_match(lambda: zz.run(states, qs, source, rank, P, True, wl.scale, finalize_outs=outs),
                   zz.emu.copy if staging == "side" else None, compute, [t for pair in outs for t in pair])


@pytest.mark.parametrize("staging", ["side", "fused"])
@pytest.mark.parametrize("rank", [0, 1, 3])
def test_captured_zigzag_block_ring_replays_bit_identically(staging, rank):
    """ZigzagRing.run_block (whole blocks, strided launches, per-piece splits
    for the fused init and finalize) captured and replayed: every replay and
    the eager rings between them give the eager ring's outputs bit for bit."""
    heads, d, rows, P = 2, 128, 256, 4
    wl = synth.Workload("graph_zigzag_block", 92, heads, d, rows, P, "bf16", True, (rank,))
    zw = synth.zigzag_workload(wl)
    jobs = [(r, b) for b in range(zw.blocks) for r in (synth.ROLE_Q, synth.ROLE_K, synth.ROLE_V)]
    host = gen_blocks(zw, jobs)
    dev = {key: to_device(x, zw) for key, x in host.items()}
    cat = lambda role, j: torch.cat([dev[(role, b)] for b in zigzag_blocks(j, P)], dim=2)
    q = cat(synth.ROLE_Q, rank)
    kv = {j: (cat(synth.ROLE_K, j), cat(synth.ROLE_V, j)) for j in range(P)}
    compute = torch.cuda.Stream()
    st = _lib.State(1, heads, 2 * zw.rows, d)
    zz = ZigzagRing((1, heads, zw.rows, d), q.dtype, compute_stream=compute, staging=staging)
    out = (torch.empty(st.o.shape, device="cuda"), torch.empty(st.m.shape, device="cuda"))
    _say(f"zigzag block graph rank {rank} staging {staging}")
    _replays_match(lambda: zz.run_block(st, q, lambda j: kv[j], rank, P, True, wl.scale, finalize_out=out),
                   zz.emu.copy if staging == "side" else None, compute, list(out))
