"""CPU oracle for the skew-aware MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct Python/numpy implementations of what the hot
path computes, written from the MegaFlux summary (picx.dev/p/e4jAzZ):

* ``route``  -- per-expert counts c_e, skew kappa, block counts b_e, padded
  stable slotting ("Routing Skew Problem" kappa equation; "Problem
  Formulation" block definition).
* ``plan``   -- the bounded greedy min-max placement with four searches and
  the reduction-aware backward variant ("Bounded Greedy Search"), plus a
  brute-force optimum of the min-max program ("Problem Formulation").
* ``ffn``    -- dense per-token SwiGLU expert FFN forward and its gradients
  ("Backward" section, expert-computation and gradient equations), in fp64.
* ``fp8``    -- OCP e4m3fn decoding and 128x128 block dequantisation.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``moe_expert_ffn_amd``) and imports nothing from it.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, library routines for the special cases they reduce to,
invariants, brute force and finite differences).  The greedy planner's
individual choices (tie-breaks, order, round bound) are not fixed by the
pages; they are pinned to the documented reading by hand-worked fixtures in
``tests/golden/``.
"""
