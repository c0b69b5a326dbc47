"""Seeded synthetic workloads for one rank's ring step.

This module draws random numbers and rounds them to bfloat16; it holds none of
the attention arithmetic.  The tests, the benchmark and the smoke check take
their inputs from here, so the HIP path and the CPU oracle see identical bytes.

Every block is drawn on its own from
    numpy PCG64(SeedSequence([workload_seed, role, block]))
with role 0 = Q (block = the rank), 1 = K, 2 = V, as float32 standard normals of
shape [heads, rows, head_dim] (batch 1), so a million-token workload never needs
all of its blocks on the host at once and any block can be regenerated alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

ROLE_Q, ROLE_K, ROLE_V = 0, 1, 2
ROLE_DO = 3   # gradient of the loss with respect to the output (backward inputs)


@dataclass(frozen=True)
class Workload:
    """One rank's share of a sequence split into `blocks` contiguous blocks."""
    name: str
    seed: int
    heads: int
    head_dim: int
    rows: int            # tokens per block (query rows of the rank = key rows per block)
    blocks: int          # P, blocks in the ring
    dtype: str           # "f32" or "bf16"
    causal: bool
    ranks: tuple         # ranks emulated for this workload
    rescale_stress: bool = False
    # Extreme scores: every scaled score against key `spike_key` (-1: every key)
    # of each block in `spike_blocks` is offset by `spike` (see block_f32).
    spike: float = 0.0
    spike_blocks: tuple = ()
    spike_key: int = -1
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def tokens(self) -> int:
        return self.rows * self.blocks


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32_h1_d64_c128_p4", 1, 1, 64, 128, 4, "f32", True, (1,),
                 note="run both causal and non-causal"),
        Workload("causal_bf16_h32_d128_c4096_p8", 2, 32, 128, 4096, 8, "bf16", True,
                 (0, 3, 7)),
        Workload("rescale_bf16_h8_d128_c2048_p16", 3, 8, 128, 2048, 16, "bf16", False,
                 (15,), rescale_stress=True,
                 note="every score against block j carries +2j; run in ring order and reversed"),
        Workload("longshare_bf16_h16_d64_c16384_p32", 4, 16, 64, 16384, 32, "bf16", True,
                 (31,), note="two half-rings merged"),
        Workload("million_bf16_h8_d128_c16384_p64", 5, 8, 128, 16384, 64, "bf16", True,
                 (63,), note="checked on 256 sampled query rows"),
    ]
}


def zigzag_workload(wl: Workload) -> Workload:
    """The same sequence cut into 2P sub-blocks of rows/2 tokens (the zigzag
    partition: rank i holds sub-blocks i and 2P-1-i).  Sub-block b is drawn
    from the seeded generator with block index b."""
    if wl.rows % 2:
        raise ValueError(f"{wl.name}: zigzag needs an even block length, got {wl.rows}")
    return replace(wl, name=wl.name + "_zigzag", rows=wl.rows // 2, blocks=2 * wl.blocks)


def normal_block(seed: int, role: int, block: int, heads: int, rows: int,
                 head_dim: int) -> np.ndarray:
    """float32 standard normals [heads, rows, head_dim] for one (role, block)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, role, block])))
    return rng.standard_normal((heads, rows, head_dim), dtype=np.float32)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits.

    Inputs here are finite normals, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def block_f32(wl: Workload, role: int, block: int, rows: int | None = None,
              heads: int | None = None) -> np.ndarray:
    """float32 values of one block before any bf16 rounding.

    For the rescale-stress workload every query row is re-centred to
    coordinate mean exactly 1 (so q . 1 = head_dim) and key block j is shifted
    by 2j/sqrt(head_dim) along the all-ones direction, which adds 2j to every
    scaled score against block j (up to the later bf16 rounding).

    Extreme-score workloads (spike != 0) re-centre the query rows the same way
    and shift key `spike_key` (every key if -1) of each block in spike_blocks
    by spike/sqrt(head_dim) along the all-ones direction, which offsets every
    scaled score against those keys by `spike` (up to the bf16 rounding).
    """
    rows = wl.rows if rows is None else rows
    heads = wl.heads if heads is None else heads
    z = normal_block(wl.seed, role, block, heads, rows, wl.head_dim)
    if wl.rescale_stress or wl.spike:
        if role == ROLE_Q:
            z = z - z.mean(axis=2, keepdims=True, dtype=np.float64).astype(np.float32) + 1.0
        elif role == ROLE_K and wl.rescale_stress:
            z = z + np.float32(2.0 * block / math.sqrt(wl.head_dim))
        elif role == ROLE_K and block in wl.spike_blocks:
            shift = np.float32(wl.spike / math.sqrt(wl.head_dim))
            if wl.spike_key < 0:
                z = z + shift
            elif wl.spike_key < rows:
                z[:, wl.spike_key, :] += shift
    return np.ascontiguousarray(z, dtype=np.float32)


def block(wl: Workload, role: int, block_idx: int, rows: int | None = None,
          heads: int | None = None) -> np.ndarray:
    """One block as the device receives it: float32, or bfloat16 bits (uint16)."""
    x = block_f32(wl, role, block_idx, rows, heads)
    if wl.dtype == "bf16":
        return round_to_bf16_bits(x)
    return x


def sample_rows(seed: int, rows: int, count: int) -> np.ndarray:
    """Sorted query-row sample: rows 0 and rows-1 always, the rest drawn
    without replacement from SeedSequence([seed, 99])."""
    if count >= rows:
        return np.arange(rows)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    inner = rng.choice(np.arange(1, rows - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, rows - 1], inner])).astype(np.int64)

