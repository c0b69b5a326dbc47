"""GPU parity of decoding: a short query block against P key/value shards
(ShardedDecode: local ra_step per shard with kv_rows != rows, tree of
ra_lse_merge, finalize; ChunkedDecode: one ra_step over the shards as batch
entries, one ra_merge_finalize) against the fp64 oracle over the whole cache,
and ra_merge_finalize alone against the oracle's merge and finalize.

Inputs come from ring_attention_block_amd.synth; expected values from oracle/.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import blockwise, dense
from ring_attention_block_amd import _lib, synth
from ring_attention_block_amd.decode import ShardedDecode

from _helpers import assert_close, oracle_values, to_device, tol_for

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.lib()


CASES = [
    # (heads, head_dim, query rows, shard rows, shards, dtype)
    (2, 128, 1, 4096, 8, "bf16"),
    (4, 128, 16, 1000, 3, "bf16"),
    (3, 64, 64, 200, 5, "bf16"),
    (2, 64, 5, 129, 4, "f32"),
    (1, 128, 300, 64, 2, "f32"),
    (2, 128, 7, 333, 1, "bf16"),
]


@pytest.mark.parametrize("heads,d,rq,c,P,dtype", CASES)
def test_decode_against_sharded_cache(heads, d, rq, c, P, dtype):
    # Shards are blocks 0..P-1 of a workload with c rows per block; the query
    # block is rq rows drawn as Q block P (the tokens after the cache).
    wl = synth.Workload(f"dec_{dtype}_h{heads}_d{d}_q{rq}_c{c}_p{P}", 300 + rq + c, heads, d, c,
                        P + 1, dtype, False, (P,))
    _say(wl.name)
    qh = synth.block(wl, synth.ROLE_Q, P, rows=rq)
    assert qh.shape == (heads, rq, d)
    kh = [synth.block(wl, synth.ROLE_K, j) for j in range(P)]
    vh = [synth.block(wl, synth.ROLE_V, j) for j in range(P)]
    q = to_device(qh, wl)
    kv = [(to_device(k, wl), to_device(v, wl)) for k, v in zip(kh, vh)]
    dec = ShardedDecode(q.shape, P)
    o, lse = dec.run(q, kv, wl.scale)
    torch.cuda.synchronize()
    to, tl = tol_for(wl)
    kp = np.arange(P * c)
    qp = np.full(rq, P * c)
    for hh in range(heads):
        want_o, want_lse = dense.attention(
            oracle_values(qh[hh:hh + 1], wl),
            np.concatenate([oracle_values(k[hh:hh + 1], wl) for k in kh], axis=1),
            np.concatenate([oracle_values(v[hh:hh + 1], wl) for v in vh], axis=1),
            qp, kp, False, wl.scale)
        eo = assert_close(o[0, hh].cpu().numpy(), want_o[0], to, f"head {hh} O")
        el = assert_close(lse[0, hh].cpu().numpy(), want_lse[0], tl, f"head {hh} LSE")
    _say(f"  max|dO|={eo:.2e} max|dLSE|={el:.2e} (last head)")


def test_unequal_block_step_matches_merge_of_halves():
    """One non-causal ra_step over a 2c-row key/value block agrees with the
    merge of two c-row steps; and a zero-row block leaves the state bit-identical."""
    wl = synth.Workload("dec_split", 77, 2, 128, 256, 3, "bf16", False, (2,))
    q = to_device(synth.block(wl, synth.ROLE_Q, 2, rows=40), wl)
    k = [to_device(synth.block(wl, synth.ROLE_K, j), wl) for j in range(2)]
    v = [to_device(synth.block(wl, synth.ROLE_V, j), wl) for j in range(2)]
    st = _lib.State(1, 2, 40, 128)
    _lib.state_init(st)
    _lib.step(st, q, torch.cat(k, 2).contiguous(), torch.cat(v, 2).contiguous(), 0, 0, 1, False,
              wl.scale)
    before = [t.clone() for t in (st.m, st.l, st.o)]
    empty = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    _lib.step(st, q, empty, empty, 0, 0, 1, False, wl.scale)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, (st.m, st.l, st.o)))
    o1, lse1 = _lib.finalize(st)
    dec = ShardedDecode(q.shape, 2)
    o2, lse2 = dec.run(q, list(zip(k, v)), wl.scale)
    torch.cuda.synchronize()
    # Both round P to bf16 (2^-9 relative per term), relative to different
    # reference maxima, so they agree to that rounding level, well inside the
    # oracle tolerance each of them meets.
    assert_close(o1.cpu().numpy(), o2.cpu().numpy(), 2e-3, "O whole vs merged halves")
    assert_close(lse1.cpu().numpy(), lse2.cpu().numpy(), 2e-3, "LSE whole vs merged halves")


CHUNKED = [
    # (heads, head_dim, query rows, chunk rows, chunks, dtype)
    (2, 128, 1, 512, 8, "bf16"),
    (4, 128, 16, 1000, 4, "bf16"),
    (3, 64, 64, 200, 2, "bf16"),
    (2, 64, 5, 129, 4, "f32"),
    (1, 128, 300, 64, 1, "f32"),
    (2, 128, 7, 333, 16, "bf16"),
    (2, 128, 3, 700, 3, "bf16"),
    (1, 64, 33, 96, 5, "f32"),
]


@pytest.mark.parametrize("heads,d,rq,c,n,dtype", CHUNKED)
def test_chunked_decode(heads, d, rq, c, n, dtype):
    """ChunkedDecode (the cache as n chunks along the batch axis, one ra_step
    launch over all chunks, one merge-and-finalize launch) against the oracle
    over the whole cache."""
    from ring_attention_block_amd.decode import ChunkedDecode
    wl = synth.Workload(f"cdec_{dtype}_h{heads}_d{d}_q{rq}_c{c}_n{n}", 600 + rq + c, heads, d, c,
                        n + 1, dtype, False, (n,))
    _say(wl.name)
    qh = synth.block(wl, synth.ROLE_Q, n, rows=rq)
    kh = [synth.block(wl, synth.ROLE_K, j) for j in range(n)]
    vh = [synth.block(wl, synth.ROLE_V, j) for j in range(n)]
    q = to_device(qh, wl)
    k = torch.cat([to_device(x, wl) for x in kh], dim=0).contiguous()
    v = torch.cat([to_device(x, wl) for x in vh], dim=0).contiguous()
    dec = ChunkedDecode(q.shape, n)
    for _ in range(2):   # the second call reuses the states of the first
        o, lse = dec.run(q, k, v, wl.scale)
    torch.cuda.synchronize()
    to, tl = tol_for(wl)
    kp, qp = np.arange(n * c), np.full(rq, n * c)
    for hh in range(heads):
        want_o, want_lse = dense.attention(
            oracle_values(qh[hh:hh + 1], wl),
            np.concatenate([oracle_values(x[hh:hh + 1], wl) for x in kh], axis=1),
            np.concatenate([oracle_values(x[hh:hh + 1], wl) for x in vh], axis=1),
            qp, kp, False, wl.scale)
        eo = assert_close(o[0, hh].cpu().numpy(), want_o[0], to, f"head {hh} O")
        el = assert_close(lse[0, hh].cpu().numpy(), want_lse[0], tl, f"head {hh} LSE")
    _say(f"  max|dO|={eo:.2e} max|dLSE|={el:.2e} (last head)")


@pytest.mark.parametrize("heads,d,rq,c,P,splits,dtype", [
    (2, 128, 16, 512, 4, 2, "bf16"),
    (3, 64, 1, 384, 2, 3, "bf16"),
    (2, 128, 5, 256, 3, 4, "f32"),
])
def test_chunked_decode_split_shards(heads, d, rq, c, P, splits, dtype):
    """Each shard laid out as `splits` chunks of consecutive keys
    (ring.split_keys, the layout bench.py's decode uses): ChunkedDecode over
    the P * splits chunks against the oracle over the whole cache."""
    from ring_attention_block_amd.decode import ChunkedDecode
    from ring_attention_block_amd.ring import split_keys
    wl = synth.Workload(f"sdec_{dtype}_h{heads}_d{d}_q{rq}_c{c}_p{P}_s{splits}", 700 + rq + c, heads, d,
                        c, P + 1, dtype, False, (P,))
    _say(wl.name)
    qh = synth.block(wl, synth.ROLE_Q, P, rows=rq)
    kh = [synth.block(wl, synth.ROLE_K, j) for j in range(P)]
    vh = [synth.block(wl, synth.ROLE_V, j) for j in range(P)]
    q = to_device(qh, wl)
    k = torch.cat([split_keys(to_device(x, wl), splits) for x in kh], dim=0)
    v = torch.cat([split_keys(to_device(x, wl), splits) for x in vh], dim=0)
    dec = ChunkedDecode(q.shape, P * splits)
    o, lse = dec.run(q, k, v, wl.scale)
    torch.cuda.synchronize()
    to, tl = tol_for(wl)
    kp, qp = np.arange(P * c), np.full(rq, P * c)
    for hh in range(heads):
        want_o, want_lse = dense.attention(
            oracle_values(qh[hh:hh + 1], wl),
            np.concatenate([oracle_values(x[hh:hh + 1], wl) for x in kh], axis=1),
            np.concatenate([oracle_values(x[hh:hh + 1], wl) for x in vh], axis=1),
            qp, kp, False, wl.scale)
        eo = assert_close(o[0, hh].cpu().numpy(), want_o[0], to, f"head {hh} O")
        el = assert_close(lse[0, hh].cpu().numpy(), want_lse[0], tl, f"head {hh} LSE")
    _say(f"  max|dO|={eo:.2e} max|dLSE|={el:.2e} (last head)")


MERGE_CASES = [
    # (output batch, parts, heads, rows, head_dim)
    (2, 5, 3, 37, 64),
    (1, 8, 2, 300, 128),
    (3, 1, 1, 5, 128),
    (1, 3, 4, 64, 64),
]


@pytest.mark.parametrize("out_batch,parts,heads,rows,d", MERGE_CASES)
def test_merge_finalize_against_oracle(out_batch, parts, heads, rows, d):
    """ra_merge_finalize over states that the oracle folded (some parts empty
    for some rows, one row empty in every part) against the oracle's pairwise
    merge and finalize of the same fp32-rounded states; and against
    ra_lse_merge pairs plus ra_finalize on the GPU."""
    wl = synth.Workload(f"mf_b{out_batch}_p{parts}_h{heads}_c{rows}_d{d}", 900 + rows + parts,
                        heads, d, rows, parts + 1, "f32", False, (parts,))
    _say(wl.name)
    rng_rows = np.arange(rows)
    st = _lib.State(out_batch * parts, heads, rows, d)
    parts_f32 = {}
    for b in range(out_batch):
        for h in range(heads):
            q = synth.block(wl, synth.ROLE_Q, parts, rows=rows)[h].astype(np.float64)
            for p in range(parts):
                k = synth.block(wl, synth.ROLE_K, p)[h].astype(np.float64) * (1 + b)
                v = synth.block(wl, synth.ROLE_V, p)[h].astype(np.float64)
                allowed = np.ones((rows, rows), dtype=bool)
                allowed[(rng_rows + p + b) % 4 == 0] = False     # this part misses some rows
                allowed[rows - 1] = False                        # a row no part sees
                s_blk = (q @ k.T) * wl.scale
                ost = blockwise.fold_block(blockwise.empty_state(rows, d), s_blk, v, allowed)
                m32, l32, o32 = (x.astype(np.float32) for x in (ost.m, ost.l, ost.o))
                parts_f32[(b, h, p)] = (m32, l32, o32)
                sb = b * parts + p
                st.m[sb, h] = torch.from_numpy(m32)
                st.l[sb, h] = torch.from_numpy(l32)
                st.o[sb, h] = torch.from_numpy(o32)
    o, lse = _lib.merge_finalize(st, parts)
    ob, _ = _lib.merge_finalize(st, parts, torch.bfloat16)
    torch.cuda.synchronize()
    for b in range(out_batch):
        for h in range(heads):
            acc = blockwise.empty_state(rows, d)
            for p in range(parts):
                m32, l32, o32 = parts_f32[(b, h, p)]
                acc = blockwise.merge(acc, blockwise.State(m32.astype(np.float64),
                                                           l32.astype(np.float64),
                                                           o32.astype(np.float64)))
            want_o, want_lse = blockwise.finalize(acc)
            assert_close(o[b, h].cpu().numpy(), want_o, 1e-5, f"b{b} h{h} O")
            assert_close(lse[b, h].cpu().numpy(), want_lse, 1e-5, f"b{b} h{h} LSE")
            # bf16 output: round-to-nearest-even of the fp32 result (2^-9 relative)
            assert_close(ob[b, h].float().cpu().numpy(), want_o,
                         float(np.abs(want_o).max()) * 2 ** -8 + 1e-6, f"b{b} h{h} bf16 O")
    assert bool((o[:, :, rows - 1] == 0).all()) and bool(torch.isneginf(lse[:, :, rows - 1]).all())
    # Against the pairwise merges on the GPU (rounding order differs only).
    want = []
    for b in range(out_batch):
        dst = st.batch_slice(b * parts, 1)
        for p in range(1, parts):
            _lib.lse_merge(dst, st.batch_slice(b * parts + p, 1))
        want.append(_lib.finalize(dst))
    torch.cuda.synchronize()
    for b, (wo, wlse) in enumerate(want):
        assert_close(o[b].cpu().numpy(), wo[0].cpu().numpy(), 1e-5, f"b{b} O vs pairwise")
        assert_close(lse[b].cpu().numpy(), wlse[0].cpu().numpy(), 1e-5, f"b{b} LSE vs pairwise")


@pytest.mark.parametrize("dtype,d,rows,kv_rows,chunks,heads",
                         [("bf16", 128, 16, 4096, 8, 32), ("bf16", 64, 300, 129, 3, 2),
                          ("bf16", 128, 1000, 512, 2, 4), ("f32", 64, 5, 200, 4, 2)])
def test_query_broadcast_is_bit_identical(dtype, d, rows, kv_rows, chunks, heads):
    """ra_step with RA_STEP_Q_BROADCAST (one query block for every batch entry)
    gives exactly what the same step gives with the query block repeated along
    the batch, with and without the fresh and finalize flags."""
    wl = synth.Workload(f"qbc_{dtype}_d{d}_q{rows}_c{kv_rows}_n{chunks}", 950 + rows, heads, d, kv_rows,
                        chunks + 1, dtype, False, (chunks,))
    _say(wl.name)
    q1 = to_device(synth.block(wl, synth.ROLE_Q, chunks, rows=rows), wl)
    k = torch.cat([to_device(synth.block(wl, synth.ROLE_K, j), wl) for j in range(chunks)]).contiguous()
    v = torch.cat([to_device(synth.block(wl, synth.ROLE_V, j), wl) for j in range(chunks)]).contiguous()
    qn = q1.expand(chunks, -1, -1, -1).contiguous()
    for flags in (0, _lib.RA_STEP_FRESH, _lib.RA_STEP_FRESH | _lib.RA_STEP_FINALIZE):
        res = []
        for q, extra in ((qn, 0), (q1, _lib.RA_STEP_Q_BROADCAST)):
            st = _lib.State(chunks, heads, rows, d)
            _lib.state_init(st)
            o = torch.full(st.o.shape, float("nan"), device="cuda")
            lse = torch.full(st.m.shape, float("nan"), device="cuda")
            _lib.step(st, q, k, v, 0, 0, 1, False, wl.scale, flags=flags | extra, o_out=o,
                      lse_out=lse)
            torch.cuda.synchronize()
            res.append([t.clone() for t in (st.m, st.l, st.o, o, lse)])
        for a, b in zip(*res):
            assert torch.equal(a.nan_to_num(7.0), b.nan_to_num(7.0)), f"flags={flags}"
