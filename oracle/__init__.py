"""CPU oracle for deduplicated paged decode attention -- TEST INFRASTRUCTURE.

This package is the plain, slow, obviously correct statement of what the device
path computes.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it.  The product path never routes through it,
and it shares no code with the library: it imports only numpy and the seeded
input generator (``workload``).

Modules and the passages they follow:

* ``dedup``     -- block fingerprint + refcount + copy-on-write bookkeeping
  (INMS walkthrough, sec. 2.2 and sec. 3.2), content-indexed segments (TokenDance
  write-up, sec. 1 "round-aware prompt interface"), master/mirror block-sparse
  deltas (TokenDance write-up, sec. 3).  Exact keys, no hashing.
* ``rope``      -- RoPE offset compensation: the rotation that moves a stored
  key from position a to b depends on b - a only; V is not rotated (INMS
  walkthrough, sec. 2.3 and sec. 3.2).
* ``q4``        -- groupwise 4-bit dequantisation x = s*c + z (Q4 KV paper
  summary, sec. 2.1; group 64 with fp16 scale and zero).
* ``attention`` -- dense materialisation per agent and softmax attention with
  scale 1/sqrt(head_dim) (MemDecay blog, sec. 4.2), in float64.
* ``lifecycle`` -- decode-time append with copy-on-write, sequence destroy, and
  the reference-leak audit with forced reclamation (INMS walkthrough, sec. 2.2,
  sec. 3.3 and sec. 5.3), with a content model for decode after appends.
* ``mirror``    -- master/mirror diff flags and the fused restore of a mirror's
  blocks (TokenDance write-up, sec. 3): delta else master, keys moved to the
  agent's positions, padding zero.
* ``persist``   -- the saved image of an agent's Q4 blocks and its reload into
  the pool (Q4 KV paper summary, sec. 2.1 and 2.2).
* ``footprint`` -- the INMS footprint closed form (INMS walkthrough, sec. 1.2)
  and per-token KV byte formulas (INMS sec. 1.2; shared-memory prefix cache
  blog, sec. 1.1).

Every function here is pinned by ``tests/test_oracle_*.py``,
``tests/test_lifecycle_cpu.py``, ``tests/test_mirror_cpu.py`` and
``tests/test_persist_cpu.py`` against closed
forms, printed worked examples (``tests/golden``), invariants or brute force.
"""
