"""GPU parity sweep: seeded random folds through the C ABI against the fp64 oracle.

Each case draws from its own seed:
- batch (1-3), heads (1-5), head_dim (64 or 128), input dtype (bf16 or fp32);
- query rows (1-700) and the number of visited blocks P (1-4);
- causal or not; a non-causal case gives its key/value blocks a length of
  their own (kv_rows != rows, as a decode step against a cache shard does);
- the rank i and a random visiting order of the P blocks;
- whether the first and last launched steps fuse the state initialisation
  (RA_STEP_FRESH) and the finalisation (RA_STEP_FINALIZE), and the output
  dtype (fp32 or bf16);
- for batch > 1, whether the query block is shared along the batch
  (RA_STEP_Q_BROADCAST).

The expected O and LSE come from oracle.dense over the visited blocks: the
online-softmax fold gives dense softmax attention in any block order (Ring
Attention Math Deep, "The online-softmax identity that makes streaming
legal"), and the causal case of each step (skip, diagonal, full) follows
"Ring Attention：把超长序列沿设备环流动", section "Causal Attention
让环不再完全对称".
Tolerances: max abs error, fp32 inputs 1e-5 on O and LSE, bf16 inputs 2e-2 / 5e-3; a bf16
output takes the bf16 tolerance on O.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import dense
from ring_attention_block_amd import _lib, synth

from _helpers import BF16_TOL, F32_TOL, assert_close, oracle_values, to_device

pytestmark = pytest.mark.gpu

N_CASES = 40


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.lib()


def draw_case(n):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([4242, n])))
    c = dict(
        batch=int(rng.integers(1, 4)), heads=int(rng.integers(1, 6)),
        d=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "bf16", "f32"])),
        rows=int(rng.choice([1, 31, 64, 65, 127, 200, 256, 300, 511, 700])),
        P=int(rng.integers(1, 5)), causal=bool(rng.random() < 0.5),
        fused=bool(rng.random() < 0.5), out_bf16=bool(rng.random() < 0.3))
    c["kv_rows"] = c["rows"] if c["causal"] else int(rng.choice([1, 63, 64, 100, 257, 640]))
    c["rank"] = int(rng.integers(0, c["P"]))
    c["order"] = [int(x) for x in rng.permutation(c["P"])]
    c["qbc"] = c["batch"] > 1 and bool(rng.random() < 0.5)
    return c


def _dev(x, wl, batch, heads):
    t = to_device(x, wl)                               # [1, batch*heads, n, d]
    return t.reshape(batch, heads, *t.shape[2:]).contiguous()


@pytest.mark.parametrize("n", range(N_CASES))
def test_random_fold_sequence(n):
    c = draw_case(n)
    print(f"sweep case {n}: {c}", flush=True)
    sys.stdout.flush()
    B, H, d, R, N, P = c["batch"], c["heads"], c["d"], c["rows"], c["kv_rows"], c["P"]
    qb = 1 if c["qbc"] else B
    wq = synth.Workload(f"sweep{n}_q", 7000 + n, qb * H, d, R, P, c["dtype"], c["causal"], (c["rank"],))
    wk = synth.Workload(f"sweep{n}_kv", 8000 + n, B * H, d, N, P, c["dtype"], c["causal"], ())
    scale = wq.scale
    q_np = synth.block(wq, synth.ROLE_Q, c["rank"])
    kv_np = {j: (synth.block(wk, synth.ROLE_K, j), synth.block(wk, synth.ROLE_V, j)) for j in range(P)}
    q = _dev(q_np, wq, qb, H)
    kv = {j: (_dev(k, wk, B, H), _dev(v, wk, B, H)) for j, (k, v) in kv_np.items()}

    i, order = c["rank"], c["order"]
    launched = [j for j in order if _lib.step_case(i, j, P, c["causal"]) != _lib.RA_CASE_SKIP]
    assert launched, "every rank folds at least its own block"
    out_dtype = torch.bfloat16 if c["out_bf16"] else torch.float32
    st = _lib.State(B, H, R, d)
    base = _lib.RA_STEP_Q_BROADCAST if c["qbc"] else 0
    if c["fused"]:
        o_out = torch.full((B, H, R, d), float("nan"), device="cuda").to(out_dtype)
        lse_out = torch.full((B, H, R), float("nan"), device="cuda")
        for j in order:
            flags = base
            if j == launched[0]:
                flags |= _lib.RA_STEP_FRESH
            if j == launched[-1]:
                flags |= _lib.RA_STEP_FINALIZE
            fin = flags & _lib.RA_STEP_FINALIZE
            _lib.step(st, q, *kv[j], i, j, P, c["causal"], scale, flags=flags,
                      o_out=o_out if fin else None, lse_out=lse_out if fin else None)
        o, lse = o_out, lse_out
    else:
        _lib.state_init(st)
        for j in order:
            _lib.step(st, q, *kv[j], i, j, P, c["causal"], scale, flags=base)
        o, lse = _lib.finalize(st, out_dtype)
    torch.cuda.synchronize()

    visited = sorted(order)
    qp = dense.ring_positions(i, R)
    kp = np.concatenate([dense.ring_positions(j, N) for j in visited])
    qv = oracle_values(q_np, wq).reshape(qb, H, R, d)
    kvv = {j: (oracle_values(k, wk).reshape(B, H, N, d), oracle_values(v, wk).reshape(B, H, N, d))
           for j, (k, v) in kv_np.items()}
    tol_o, tol_l = F32_TOL if c["dtype"] == "f32" else BF16_TOL
    if c["out_bf16"]:
        tol_o = BF16_TOL[0]
    got_o = o.float().cpu().numpy()
    got_l = lse.cpu().numpy()
    for b in range(B):
        kk = np.concatenate([kvv[j][0][b] for j in visited], axis=1)
        vv = np.concatenate([kvv[j][1][b] for j in visited], axis=1)
        want_o, want_l = dense.attention(qv[0 if c["qbc"] else b], kk, vv, qp, kp, c["causal"], scale)
        assert_close(got_o[b], want_o, tol_o, f"case {n} batch {b} O")
        assert_close(got_l[b], want_l, tol_l, f"case {n} batch {b} LSE")
