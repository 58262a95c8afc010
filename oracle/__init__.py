"""Oracle for the streamed DiT forward -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation of what the weight-streamed
forward computes, written from the pages' description of vLLM-Omni's
Distributed Layerwise Offload (the aisignalhub.me release page "vLLM-Omni
releases Distributed Layerwise Offload ...", sections "Weight sharding with
AllGather reconstruction" and "Double-buffered prefetch with H2D + AllGather
overlap") and, for the block internals the pages leave open, from the DiT
adaLN-Zero block of Peebles & Xie, "Scalable Diffusion Models with
Transformers" (2023), section 3.2.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the C-ABI library and its
Python binding) never imports, links or runs anything here, and this package
imports nothing from the product: the two share no code.  The only shared
module is ``synth`` (seeded inputs, no method arithmetic).

Contents:

* ``layout``  -- per-block parameter table and flat element count.
* ``shard``   -- ceil-divided, zero-padded shards and their reconstruction.
* ``dit``     -- the DiT block and the chained forward, float64 by default.
* ``trace``   -- checker for the two-slot streaming schedule's event trace.

Every function here is pinned by ``tests/test_oracle_*.py`` (closed forms,
library routines, brute force on tiny inputs, special cases and the pages'
own figures).  The pages print no numeric example of the block math, so its
pins come from the mathematics (closed forms, library routines, special
cases) rather than from values the pages print.
"""
from . import layout, shard, dit, trace  # noqa: F401
