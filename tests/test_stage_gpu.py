"""GPU: the staging copy (ra_stage_block, ra_stage_block_ex) moves exactly the bytes asked for.

Byte-exact comparison on seeded random bytes, with guard regions around the
destination that must stay untouched.  Sizes cover a copy shorter than one
round of the workgroup's accesses, ragged tails, chunk boundaries, and blocks
large enough that every workgroup copies many rounds (a 32 MiB key block of
the 32-head workload, and more).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib

pytestmark = pytest.mark.gpu

GUARD = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _lib.lib()


@pytest.mark.parametrize("alone", [False, True], ids=["beside_step", "alone"])
@pytest.mark.parametrize("nbytes", [16, 4080, 12288, 12304, 1572864 + 16 * 7, 33554432,
                                    100 * 1048576 + 48])
def test_stage_block_copies_exactly(nbytes, alone):
    """Both grids: the small one of ra_stage_block and the full-chip one of
    ra_stage_block_ex with RA_STAGE_ALONE."""
    print(f"  stage_block {nbytes} bytes alone={alone}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(nbytes)
    src_host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    src = torch.from_numpy(src_host).cuda()
    dst_all = torch.full((nbytes + 2 * GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = dst_all[GUARD:GUARD + nbytes]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    _lib.stage_block(dst, src, stream, alone=alone)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert bool((dst_all[:GUARD] == 0xA5).all()) and bool((dst_all[GUARD + nbytes:] == 0xA5).all())
