"""Shared test plumbing: move seeded blocks to the device and compare results.

Inputs come from ring_attention_block_amd.synth (random draws only); expected
values come from oracle/ only.
"""
from __future__ import annotations

import numpy as np

from oracle import dense
from ring_attention_block_amd import synth

BF16_TOL = (2e-2, 5e-3)   # max abs error on O, LSE for bf16 inputs, fp32 accumulation
F32_TOL = (1e-5, 1e-5)


def tol_for(wl):
    return BF16_TOL if wl.dtype == "bf16" else F32_TOL


def to_device(x: np.ndarray, wl, device="cuda"):
    import torch
    if wl.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.reshape(1, *x.shape).to(device)


def oracle_values(x: np.ndarray, wl) -> np.ndarray:
    return dense.bf16_bits_to_f64(x) if wl.dtype == "bf16" else x.astype(np.float64)


def oracle_rank(wl, rank, blocks, causal, row_sel=None, head_sel=None, cache=None):
    """Oracle O [H', R', d], LSE [H', R'] for `rank` over key blocks `blocks`."""
    cache = {} if cache is None else cache

    def get(role, j):
        key = (role, j)
        if key not in cache:
            cache[key] = synth.block(wl, role, j)
        return cache[key]

    heads = range(wl.heads) if head_sel is None else head_sel
    rows = np.arange(wl.rows) if row_sel is None else np.asarray(row_sel)
    q_all = get(synth.ROLE_Q, rank)
    kp = np.concatenate([dense.ring_positions(j, wl.rows) for j in blocks])
    qp = dense.ring_positions(rank, wl.rows)[rows]
    outs, lses = [], []
    for h in heads:
        q = oracle_values(q_all[h:h + 1, rows], wl)
        k = np.concatenate([oracle_values(get(synth.ROLE_K, j)[h:h + 1], wl) for j in blocks], axis=1)
        v = np.concatenate([oracle_values(get(synth.ROLE_V, j)[h:h + 1], wl) for j in blocks], axis=1)
        o, lse = dense.attention(q, k, v, qp, kp, causal, wl.scale)
        outs.append(o[0])
        lses.append(lse[0])
    return np.stack(outs), np.stack(lses)


def assert_close(got, want, tol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    fin_g, fin_w = np.isfinite(got), np.isfinite(want)
    assert np.array_equal(fin_g, fin_w), f"{what}: finite pattern differs"
    assert np.array_equal(got[~fin_g], want[~fin_w]), f"{what}: non-finite values differ"
    if fin_g.any():
        err = float(np.max(np.abs(got[fin_g] - want[fin_w])))
        assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"
        return err
    return 0.0


def gen_blocks(wl, jobs, threads=16):
    """synth.block for each (role, block) in jobs, in a thread pool.  Each block
    has its own seed, so the values do not depend on the threading."""
    import concurrent.futures as cf
    jobs = list(jobs)
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        arrs = list(ex.map(lambda rj: synth.block(wl, *rj), jobs))
    return dict(zip(jobs, arrs))
