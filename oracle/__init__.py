"""Plain, slow CPU oracle for the DFlash draft block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in
this package.  The HIP library never calls it, and it shares no code with the
HIP library: the only module both sides read is ``synth`` (seeded inputs).

Contents:
  * ``oracle.dflash``  -- fp64 NumPy implementation of the whole hot path
    (context projection, KV injection, draft block, acceptance, session);
  * ``oracle.brute``   -- the same forward written as scalar pure-Python loops,
    for tiny shapes only, used to pin ``oracle.dflash``.

Pins (all under ``tests/``, run with ``-m "not gpu"``): brute force,
RoPE against complex multiplication, single-key and uniform-attention special
cases, context-permutation, global position-shift, block-permutation and
batch invariances, GQA == MHA with duplicated KV weights, incremental ==
one-shot projection, exhaustive acceptance enumeration, the closed form of
the expected acceptance length under independent agreement, the growth
and state-advance invariants, and the bf16 decode and round-to-nearest-even
against their definitions (hand bit patterns, every finite pattern).

Parity unpinned: whether this reading of the pages matches the exact
architecture of the trained DFlash drafters (placement of norms, the
one-position shift between block rows and proposed positions, absence of a
per-head QK norm) cannot be checked here; the pages print no intermediate
value or worked example and no checkpoint is available.
"""
