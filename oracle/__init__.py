"""CPU fp64 oracle for one rank's ring step of softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing under this package is part of the product
path: only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it.  It shares no code, header, table or helper with the
HIP library; both sides receive the same seeded inputs and nothing else.

Contents
  dense      -- the plain definition: dense masked softmax attention in fp64
                (the oracle proper).
  blockwise  -- an independent fp64 model of the online-softmax recurrence,
                the two-state merge and the final divide, used only to pin the
                dense oracle (block order, merge, skip) and to check the
                intermediate values of the worked example.
  brute      -- 50-digit decimal brute force for tiny inputs.
  backward   -- the fp64 gradients (dQ, dK, dV) of the dense forward, and the
                per-key-block contribution with probabilities recomputed from
                the saved log-sum-exp (what a ring rank accumulates).

Every function here is pinned by tests/test_oracle.py and
tests/test_oracle_backward.py against values fixed by the pages or by
mathematics; none is "parity unpinned".
"""
