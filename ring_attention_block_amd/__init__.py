"""MI355X-native ring-step attention.

One rank's ring step of softmax attention as hand-written HIP for gfx950 behind
a C ABI (include/ra.h).  Python modules here only marshal arguments:

  synth  -- seeded synthetic workloads (random draws and bf16 rounding only)
  _lib   -- ctypes binding of the C ABI (loads libra.so built in-tree)
  ring   -- single-GPU emulation of one rank's ring: side-stream staging of the
            next key/value block with double-buffered swaps

Importing this package loads nothing; the shared library is opened on first use
and a missing or unbuilt library raises immediately.
"""
