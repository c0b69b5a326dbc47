"""GPU: staging carried by the step launch (ra_step_staged, RingEmulator with
staging="fused").

The receive of the next key/value block into the free buffer while the current
block is folded ("Ring Attention Paper Breakdown: Blockwise Distributed
Transformers for Near-Infinite Context", section 2) is done by the step
kernel's own workgroups.  Checked here:
- a staged step copies exactly the bytes asked for (guard bytes around every
  destination stay untouched) and folds bit-identically to the same step
  without copies, on 8- and 4-wavefront grids, full and diagonal blocks,
  ragged lengths, idle wavefronts, head_dim 64 and 128, fp32 inputs, fused
  initialisation and finalisation;
- a step that folds nothing (a skipped causal block, an empty key block)
  still makes its copies;
- whole rings with fused staging equal the side-stream rings bit for bit
  (contiguous causal ranks at the 32-head, 4096-row shape, key ranges of a
  non-causal ring, the zigzag partition), also when every released buffer is
  filled with NaN before it is refilled, and one against the oracle.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.ring import RingEmulator, ZigzagRing, split_keys, zigzag_blocks

from _helpers import BF16_TOL, assert_close, oracle_rank

pytestmark = pytest.mark.gpu

GUARD = 4096


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.lib()


def _copies(sizes, seed):
    """(dst, src, dst_with_guards) per size: seeded random source bytes, a
    destination inside a 0xA5-filled buffer with guard bytes on both sides."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    out = []
    for n in sizes:
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()
        full = torch.full((n + 2 * GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
        out.append((full[GUARD:GUARD + n], src, full))
    return out


def _check_copies(cps):
    for dst, src, full in cps:
        n = dst.numel()
        assert torch.equal(dst, src), f"copy of {n} bytes differs"
        assert bool((full[:GUARD] == 0xA5).all()) and bool((full[GUARD + n:] == 0xA5).all()), \
            f"copy of {n} bytes wrote outside its destination"


def _state_like(st):
    s2 = _lib.State(*st.shape)
    s2.m.copy_(st.m)
    s2.l.copy_(st.l)
    s2.o.copy_(st.o)
    return s2


def _same_state(a, b):
    return torch.equal(a.m, b.m) and torch.equal(a.l, b.l) and torch.equal(a.o, b.o)


STEPS = [
    # (heads, d, rows, kv_rows, causal, i, j, dtype, flags, copy sizes)
    (32, 128, 2048, 2048, True, 1, 0, "bf16", 0, [16 << 20, 16 << 20]),        # 8 waves, full
    (32, 128, 2048, 2048, True, 1, 1, "bf16", 0, [16 << 20, 16 << 20]),        # 8 waves, diagonal
    (8, 128, 2048, 2048, False, 3, 1, "bf16", 0, [4 << 20, 4 << 20]),          # 4 waves
    (8, 128, 2048, 1024, False, 0, 5, "bf16", _lib.RA_STEP_Q_BROADCAST, [2 << 20, (1 << 20) + 48]),
    (3, 64, 200, 200, True, 2, 2, "bf16", 0, [16, 4096 * 3 + 16]),              # ragged, d 64
    (1, 128, 64, 64, False, 0, 0, "bf16", 0, [32 << 20]),                       # one workgroup, one tile
    (2, 128, 100, 333, False, 0, 0, "bf16", 0, [48, 1 << 20]),                  # idle waves, ragged keys
    (16, 64, 4096, 4096, True, 1, 1, "bf16", _lib.RA_STEP_FRESH, [8 << 20, 8 << 20]),
    (32, 128, 2048, 2048, True, 1, 0, "bf16", _lib.RA_STEP_FINALIZE, [16 << 20, 16 << 20]),
    (2, 128, 300, 300, True, 1, 0, "f32", 0, [4096, 8192]),                     # fp32: copy kernels
]


@pytest.mark.parametrize("case", range(len(STEPS)))
def test_staged_step_copies_and_folds_bit_identically(case):
    H, d, R, N, causal, i, j, dtype, flags, sizes = STEPS[case]
    _say(f"staged step case {case}: heads={H} d={d} rows={R} kv_rows={N} causal={causal} "
         f"i={i} j={j} {dtype} flags={flags} copies={sizes}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    torch.manual_seed(case)
    B = 2 if flags & _lib.RA_STEP_Q_BROADCAST else 1
    q = torch.randn(1, H, R, d, device="cuda").to(tdt)
    k = torch.randn(B, H, N, d, device="cuda").to(tdt)
    v = torch.randn(B, H, N, d, device="cuda").to(tdt)
    st = _lib.State(B, H, R, d)
    _lib.state_init(st)
    _lib.step(st, q if B == 1 else q, k, v, i, j, max(i, j) + 1, False, d ** -0.5,
              flags=flags & _lib.RA_STEP_Q_BROADCAST)       # a non-trivial starting state
    ref_st = _state_like(st)
    fin = bool(flags & _lib.RA_STEP_FINALIZE)
    outs = [(torch.full((B, H, R, d), float("nan"), device="cuda"),
             torch.full((B, H, R), float("nan"), device="cuda")) for _ in range(2)]
    torch.cuda.synchronize()
    P = max(i, j) + 1
    _lib.step(ref_st, q, k, v, i, j, P, causal, d ** -0.5, flags=flags,
              o_out=outs[0][0] if fin else None, lse_out=outs[0][1] if fin else None)
    cps = _copies(sizes, 100 + case)
    _lib.step_staged(st, q, k, v, i, j, P, causal, d ** -0.5, [(c[0], c[1]) for c in cps], flags=flags,
                     o_out=outs[1][0] if fin else None, lse_out=outs[1][1] if fin else None)
    torch.cuda.synchronize()
    _check_copies(cps)
    assert _same_state(st, ref_st), "the staged step's state differs from the plain step's"
    if fin:
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_staged_step_that_folds_nothing_still_copies():
    torch.manual_seed(7)
    q, k, v = (torch.randn(1, 4, 256, 128, device="cuda").to(torch.bfloat16) for _ in range(3))
    st = _lib.State(1, 4, 256, 128)
    _lib.state_init(st)
    _lib.step(st, q, k, v, 0, 0, 2, True, 0.1)
    before = _state_like(st)
    cps = _copies([1 << 20, 4096 + 16], 3)
    # causal future block: skipped
    _lib.step_staged(st, q, k, v, 0, 1, 2, True, 0.1, [(c[0], c[1]) for c in cps])
    torch.cuda.synchronize()
    _check_copies(cps)
    assert _same_state(st, before)
    # an empty key/value block (non-causal)
    cps = _copies([65536], 4)
    e = torch.empty(1, 4, 0, 128, device="cuda", dtype=torch.bfloat16)
    _lib.step_staged(st, q, e, e, 0, 1, 2, False, 0.1, [(c[0], c[1]) for c in cps])
    torch.cuda.synchronize()
    _check_copies(cps)
    assert _same_state(st, before)


WL = synth.WORKLOADS["causal_bf16_h32_d128_c4096_p8"]


def _blocks(wl, n, heads, rows, d, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return {j: (torch.randn(1, heads, rows, d, device="cuda", generator=g).to(dtype),
                torch.randn(1, heads, rows, d, device="cuda", generator=g).to(dtype)) for j in range(n)}


def _ring(staging, q, kv, rank, P, causal, scale, key_split=1, poison=False, timed=False):
    shape = kv[0][0].shape
    emu = RingEmulator(shape, q.dtype, staging=staging)
    if poison:
        for buf in emu.bufs:
            for t in buf:
                t.fill_(float("nan"))

        def hook(tensors, stream):
            with torch.cuda.stream(stream):
                for t in tensors:
                    t.fill_(float("nan"))
        emu.free_hook = hook
    B = key_split
    H, c, d = q.shape[1], q.shape[2], q.shape[3]
    st = _lib.State(B, H, c, d)
    o = torch.full((1, H, c, d), float("nan"), device="cuda", dtype=torch.bfloat16)
    lse = torch.full((1, H, c), float("nan"), device="cuda")
    timers = [] if timed else None
    cases = emu.run(st, q, lambda j: kv[j], rank, P, causal, scale, finalize_out=(o, lse),
                    key_split=key_split, step_timers=timers)
    torch.cuda.synchronize()
    return o, lse, cases


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_fused_ring_equals_side_ring_headline_shape(rank):
    _say(f"fused vs side ring, 32 heads x 4096 rows, rank {rank}")
    H, c, d = WL.heads, WL.rows, WL.head_dim
    kv = _blocks(WL, WL.blocks, H, c, d, 11)
    q = torch.randn(1, H, c, d, device="cuda").to(torch.bfloat16)
    o1, l1, _ = _ring("side", q, kv, rank, WL.blocks, True, WL.scale, timed=True)
    o2, l2, _ = _ring("fused", q, kv, rank, WL.blocks, True, WL.scale, timed=True)
    o3, l3, _ = _ring("fused", q, kv, rank, WL.blocks, True, WL.scale, poison=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_fused_key_split_ring_equals_side_ring():
    wl = synth.WORKLOADS["rescale_bf16_h8_d128_c2048_p16"]
    H, c, d, P = wl.heads, wl.rows, wl.head_dim, wl.blocks
    kv = {j: (split_keys(k, 2), split_keys(v, 2)) for j, (k, v) in _blocks(wl, P, H, c, d, 12).items()}
    q = torch.randn(1, H, c, d, device="cuda").to(torch.bfloat16)
    o1, l1, _ = _ring("side", q, kv, P - 1, P, False, wl.scale, key_split=2)
    o2, l2, _ = _ring("fused", q, kv, P - 1, P, False, wl.scale, key_split=2, poison=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fused_zigzag_ring_equals_side_ring():
    H, c, d, P = 8, 1024, 128, 4
    half = c // 2
    g = torch.Generator(device="cuda").manual_seed(13)
    sub = {b: tuple(torch.randn(1, H, half, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
           for b in range(2 * P)}
    rank = 1
    mine = zigzag_blocks(rank, P)

    def source(j):
        a, b = zigzag_blocks(j, P)
        return (sub[a][1], sub[b][1], sub[a][2], sub[b][2])

    res = []
    for staging in ("side", "fused"):
        zz = ZigzagRing((1, H, half, d), torch.bfloat16, staging=staging)
        sts = [_lib.State(1, H, half, d) for _ in range(2)]
        outs = [(torch.empty(1, H, half, d, device="cuda"), torch.empty(1, H, half, device="cuda")) for _ in range(2)]
        zz.run(sts, [sub[mine[0]][0], sub[mine[1]][0]], source, rank, P, True, d ** -0.5, finalize_outs=outs)
        torch.cuda.synchronize()
        res.append(outs)
    for (oa, la), (ob, lb) in zip(*res):
        assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_fused_ring_against_oracle():
    wl = synth.Workload("fused_small_bf16_h4_d128_c300_p4", 77, 4, 128, 300, 4, "bf16", True, (2,))
    from _helpers import gen_blocks, to_device
    rank = 2
    jobs = [(synth.ROLE_Q, rank)] + [(r, j) for j in range(wl.blocks) for r in (synth.ROLE_K, synth.ROLE_V)]
    cache = gen_blocks(wl, jobs)
    q = to_device(cache[(synth.ROLE_Q, rank)], wl)
    kv = {j: (to_device(cache[(synth.ROLE_K, j)], wl), to_device(cache[(synth.ROLE_V, j)], wl))
          for j in range(wl.blocks)}
    o, lse, _ = _ring("fused", q, kv, rank, wl.blocks, True, wl.scale)
    want_o, want_l = oracle_rank(wl, rank, list(range(wl.blocks)), True, cache=cache)
    assert_close(o[0].float().cpu().numpy(), want_o, BF16_TOL[0], "fused ring O")
    assert_close(lse[0].cpu().numpy(), want_l, BF16_TOL[1], "fused ring LSE")
