"""Float64 CPU oracle for the ReplaySSM decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the
``linear_recurrence_amd`` package, its HIP kernels or its C ABI) may import,
call, link or execute anything in this package.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

The oracle is written from the method as the pages describe it:

* vLLM #48018 "[Kernel] ReplaySSM: cache SSM inputs for faster Mamba2
  standard decode" (Motivation; Implementation items 1 and 3; key source
  snippet of ``mamba_mixer2.py``; Risks item 2),
* sglang #28451, the GDN/KDA ReplaySSM decode report (Motivation;
  Implementation items 1-3; Risks),
* sglang #28695 "[GDN] Support ReplaySSM Ring Spec-Verify" (memory-pool
  snippet: ring contents d, k, g).

Everything is plain NumPy in float64: loops over decode steps and over batch
rows, einsum/matmul as the only library primitives.  It shares no code with
the HIP path.  Pins that tie each function to something other than itself
(closed forms, invariants, library routines, brute force) live in
``tests/test_oracle_*.py``.

Modules
-------
``numerics``  storage rounding (fp32, bf16 round-to-nearest-even), softplus.
``mamba2``    standard selective state update (the recurrence) and the
              ReplaySSM ring replay with flush, cursor advance and ring reset.
``gdn``       gated delta rule: recurrence and ring replay.
``metadata``  host cursors of a step from token positions (decode base).
``gdn_spec``  GDN speculative verify over drafts and commit with exact fold.
``kda``       gated delta rule with a per-key-channel gate (KDA): recurrence
              and ring replay.
"""

from . import numerics, mamba2, gdn, metadata, gdn_spec, kda  # noqa: F401
