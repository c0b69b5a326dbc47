"""GPU parity of the strided step (ra_step_strided) and of the zigzag ring on
whole blocks (ZigzagRing.run_block) that it serves.

Under the zigzag partition ("Ring Attention Paper Breakdown: Blockwise
Distributed Transformers for Near-Infinite Context", section 5; "Ring
Attention：把超长序列沿设备环流动", section "Causal Attention 让环不再完全对称")
rank i holds pieces i and 2P-1-i; run_block keeps both in one block in
position order and folds each visit as row ranges of such blocks.  The strided
step is checked bit for bit against the same step on packed copies of its
operands (same kernel, same arithmetic, only the addressing differs), with the
rows outside its ranges left untouched; the ring against the fp64 oracle at
every piece's global positions (inputs from ring_attention_block_amd.synth,
expected values from oracle/ only).
"""
import sys
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.ring import ZigzagRing, zigzag_blocks, zigzag_fused_launches

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


def _rand(shape, dtype, gen):
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype).cuda()


def _state_like(st_shape, gen):
    """A non-empty state with finite, varied values (m, positive l, O)."""
    b, h, r, d = st_shape
    st = _lib.State(b, h, r, d)
    st.m.copy_(torch.randn((b, h, r), generator=gen).cuda())
    st.l.copy_(torch.rand((b, h, r), generator=gen).cuda() * 4 + 0.5)
    st.o.copy_(torch.randn((b, h, r, d), generator=gen).cuda())
    return st


CASES = [
    # (dtype, head_dim, batch, heads, block rows, query range, key block rows, key range, diagonal)
    ("bf16", 128, 2, 3, 400, (200, 200), 400, (0, 200), False),
    ("bf16", 128, 1, 4, 512, (256, 256), 512, (0, 512), False),
    ("bf16", 64, 2, 2, 258, (0, 258), 520, (131, 258), False),
    ("f32", 128, 1, 3, 300, (100, 150), 300, (0, 300), False),
    ("f32", 64, 2, 2, 128, (64, 64), 256, (64, 128), False),
    ("bf16", 128, 2, 3, 400, (200, 200), 400, (200, 200), True),
    ("bf16", 64, 1, 2, 258, (129, 129), 258, (129, 129), True),
    ("f32", 128, 1, 2, 200, (0, 100), 200, (0, 100), True),
]


@pytest.mark.parametrize("dtype,d,B,H,R,qr,KR,kr,diag", CASES)
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_strided_step_is_bit_identical_to_packed(dtype, d, B, H, R, qr, KR, kr, diag, flags):
    gen = torch.Generator().manual_seed(zlib.crc32(repr((dtype, d, B, H, R, qr, kr, diag, flags)).encode()))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = _rand((B, H, R, d), tdt, gen)
    k = _rand((B, H, KR, d), tdt, gen)
    v = _rand((B, H, KR, d), tdt, gen)
    st = _state_like((B, H, R, d), gen)
    before = [t.clone() for t in (st.m, st.l, st.o)]
    lo, n = qr
    klo, kn = kr
    o_out = torch.full((B, H, R, d), float("nan"), device="cuda")
    lse_out = torch.full((B, H, R), float("nan"), device="cuda")
    scale = d ** -0.5
    args = (0, 0, 1, diag, scale)
    view = st.row_slice(lo, n)
    _say(f"strided {dtype} d{d} B{B} H{H} rows [{lo},{lo + n}) of {R}, keys [{klo},{klo + kn}) "
         f"of {KR} diag={diag} flags={flags}")
    _lib.step_strided(view, q[:, :, lo:lo + n], k[:, :, klo:klo + kn], v[:, :, klo:klo + kn],
                      *args, flags=flags, o_out=o_out[:, :, lo:lo + n], lse_out=lse_out[:, :, lo:lo + n])
    # the same step on packed copies
    ref = _lib.State(B, H, n, d)
    for dst, src in ((ref.m, before[0]), (ref.l, before[1]), (ref.o, before[2])):
        dst.copy_(src[:, :, lo:lo + n])
    ro = torch.full((B, H, n, d), float("nan"), device="cuda")
    rl = torch.full((B, H, n), float("nan"), device="cuda")
    _lib.step(ref, q[:, :, lo:lo + n].contiguous(), k[:, :, klo:klo + kn].contiguous(),
              v[:, :, klo:klo + kn].contiguous(), *args, flags=flags, o_out=ro, lse_out=rl)
    torch.cuda.synchronize()
    outside = torch.ones(R, dtype=torch.bool, device="cuda")
    outside[lo:lo + n] = False
    for t, b, r in ((st.m, before[0], ref.m), (st.l, before[1], ref.l), (st.o, before[2], ref.o)):
        assert torch.equal(t[:, :, ~outside], r), "rows in range differ from the packed step"
        assert torch.equal(t[:, :, outside], b[:, :, outside]), "rows outside the range changed"
    if flags & _lib.RA_STEP_FINALIZE:
        assert torch.equal(o_out[:, :, lo:lo + n], ro) and torch.equal(lse_out[:, :, lo:lo + n], rl)
    assert torch.isnan(o_out[:, :, outside]).all() and torch.isnan(lse_out[:, :, outside]).all()


def _block(dev, role, pieces):
    return torch.cat([dev[(role, b)] for b in pieces], dim=2)


def run_block_ring(sub, rank, P, causal, dev, fused, staging):
    mine = zigzag_blocks(rank, P)
    q = _block(dev, synth.ROLE_Q, mine)
    kv = {j: (_block(dev, synth.ROLE_K, zigzag_blocks(j, P)),
              _block(dev, synth.ROLE_V, zigzag_blocks(j, P))) for j in range(P)}
    st = _lib.State(1, sub.heads, 2 * sub.rows, sub.head_dim)
    ring = ZigzagRing((1, sub.heads, sub.rows, sub.head_dim), q.dtype, staging=staging)
    if fused:
        out = (torch.full((1, sub.heads, 2 * sub.rows, sub.head_dim), float("nan"), device="cuda"),
               torch.full((1, sub.heads, 2 * sub.rows), float("nan"), device="cuda"))
        ring.run_block(st, q, lambda j: kv[j], rank, P, causal, sub.scale, finalize_out=out)
    else:
        ring.run_block(st, q, lambda j: kv[j], rank, P, causal, sub.scale)
        out = _lib.finalize(st, torch.float32, ring.compute)
    torch.cuda.synchronize()
    return out


SMALL = [
    # (heads, head_dim, rows per rank, ranks, dtype): pieces of rows/2, ragged tails
    (2, 128, 400, 3, "bf16"),
    (1, 64, 128, 4, "f32"),
    (3, 64, 258, 2, "bf16"),
    (2, 128, 1024, 4, "bf16"),
]


@pytest.mark.parametrize("heads,d,rows,P,dtype", SMALL)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("fused,staging", [(False, "side"), (True, "side"), (True, "fused")])
def test_zigzag_block_every_rank(heads, d, rows, P, dtype, causal, fused, staging):
    wl = synth.Workload(f"zzb_{dtype}_h{heads}_d{d}_c{rows}_p{P}", 200 + rows + d, heads, d, rows,
                        P, dtype, causal, tuple(range(P)))
    sub = synth.zigzag_workload(wl)
    cache = gen_blocks(sub, [(r, b) for b in range(2 * P)
                             for r in (synth.ROLE_Q, synth.ROLE_K, synth.ROLE_V)])
    dev = {key: to_device(x, sub) for key, x in cache.items()}
    to, tl = tol_for(sub)
    h = sub.rows
    for rank in range(P):
        launches = sum(len(ls) for _, ls in zigzag_fused_launches(rank, P, causal))
        _say(f"{sub.name} causal={causal} fused={fused} staging={staging} rank={rank} "
             f"({launches} launches)")
        o, lse = run_block_ring(sub, rank, P, causal, dev, fused, staging)
        for n, piece in enumerate(zigzag_blocks(rank, P)):
            want_o, want_lse = oracle_rank(sub, piece, range(2 * P), causal, cache=cache)
            what = f"{sub.name} causal={causal} rank {rank} piece {piece}"
            eo = assert_close(o[0, :, n * h:(n + 1) * h].cpu().numpy(), want_o, to, what + " O")
            el = assert_close(lse[0, :, n * h:(n + 1) * h].cpu().numpy(), want_lse, tl, what + " LSE")
            _say(f"  {what}: max|dO|={eo:.2e} max|dLSE|={el:.2e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rank", [63, 0])
def test_zigzag_block_million_tokens_sampled_rows(rank):
    """The million-token sequence (8 heads, d = 128, 64 ranks x 16384 tokens)
    under the zigzag partition as bench.py runs it (whole blocks, one strided
    launch per visit, fused init and finalize, side staging): ranks 63 and 0,
    64 sampled rows of each piece and every head against the oracle over all
    keys before them."""
    wl = synth.WORKLOADS["million_bf16_h8_d128_c16384_p64"]
    sub = synth.zigzag_workload(wl)
    P = wl.blocks
    mine = zigzag_blocks(rank, P)
    _say(f"{sub.name} rank {rank}: generating {2 * P} pieces")
    cache = gen_blocks(sub, [(synth.ROLE_Q, b) for b in mine] +
                       [(r, b) for b in range(2 * P) for r in (synth.ROLE_K, synth.ROLE_V)])
    dev = {key: to_device(x, sub) for key, x in cache.items()}
    o, lse = run_block_ring(sub, rank, P, True, dev, True, "side")
    del dev
    to, tl = tol_for(sub)
    rows = synth.sample_rows(wl.seed, sub.rows, 64)
    h = sub.rows
    for n, piece in enumerate(mine):
        keys = range(piece + 1)   # causal: every piece up to this one
        parts = []
        for hh in range(sub.heads):
            parts.append(oracle_rank(sub, piece, keys, True, row_sel=rows, head_sel=[hh], cache=cache))
            _say(f"  piece {piece}: oracle head {hh} over {len(keys)} pieces")
        want_o = np.concatenate([p_[0] for p_ in parts])
        want_lse = np.concatenate([p_[1] for p_ in parts])
        got_o = o[0, :, n * h:(n + 1) * h].cpu().numpy()[:, rows]
        got_l = lse[0, :, n * h:(n + 1) * h].cpu().numpy()[:, rows]
        what = f"{sub.name} rank {rank} piece {piece}, {len(rows)} rows"
        eo = assert_close(got_o, want_o, to, what + " O")
        el = assert_close(got_l, want_lse, tl, what + " LSE")
        _say(f"  {what}: max|dO|={eo:.2e} max|dLSE|={el:.2e}")
