"""Plain, slow CPU oracle for absorbed-MLA decoding.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may import,
call or execute anything in this package: only the tests, the package-level
``smoke()`` check and the ``cpu_baseline`` leg of the benchmark use it.  It
shares no code with the HIP path (no kernels, headers, helpers or tables).

Everything here is numpy in float64 (or exact integer arithmetic), written from
the pages that describe the method:

* ``attention``  -- the decode definition (dense paged cache, DSA top-k gather,
  FP8 cache), a loop-only brute force, the streaming online-softmax recurrence
  and the split merge;
* ``numerics``   -- bfloat16 / float8_e4m3fn decoding and bfloat16 rounding;
* ``fp8cache``   -- the 656-byte FP8 latent-cache record and its dequantisation;
* ``sched``      -- the split-KV tile-scheduler specification (our own: the
  pages only say the scheduler balances work, so this one is "parity unpinned"
  by the pages and pinned by invariants and brute force instead).
"""

from . import numerics, fp8cache, attention, sched  # noqa: F401
