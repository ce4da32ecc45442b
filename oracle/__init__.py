"""Plain, slow fp64 CPU oracle for the Hybrid SWA attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
module and the CPU-baseline leg of the benchmark may import this package.
The product path (the HIP library and its Python binding) never imports it,
and this package imports nothing from the product path.

Sources (the pages the method is taken from):

* "MiMo-V2.5 Series Inference Full-Link Optimization: Pushing Hybrid SWA
  Efficiency to the Extreme" (mimo.mi.com) -- section 1.1 (layer mix, window
  W = 128, compute ratio), section 1.2 (KV storage ratio), section 2.1
  "KVCache Dual Pool" (Full pool O(N), SWA pool O(W), Full index
  authoritative with a Full-to-SWA map, joint capacity check) and "SWA-aware
  prefix cache tree", point 2 (out-of-window SWA release at each prefill
  chunk and during decode).
* "Following the Bottleneck: Optimizing MiniMax M3 on AMD Instinct MI355X"
  (vLLM blog), section 3 "Which bytes move?" -- 16-token KV pages addressed
  through a page table.

Modules:

* ``attention`` -- the attention definition with explicit window masks over
  contiguous per-sequence K/V.
* ``pool``      -- the dual-pool slot bookkeeping (Full pages, SWA ring,
  Full-to-SWA map, eviction) as a plain Python simulator.
* ``closed_forms`` -- scored-pair and resident-KV counts and their ratios.
* ``transfer``  -- which positions a window-masked tier transfer moves and
  the packed host image it produces.
* ``fp8``       -- FP8 (e4m3) KV quantization per token, head and tile with
  fp32 scales, and its dequantized values.

Every function in these modules is pinned by ``tests/test_oracle*.py`` to
something other than itself (library routines, brute force, closed forms,
hand-worked fixtures); ``tests/test_oracle_mutants.py`` plants mistakes in
copies of these modules and checks that the pins catch them.  The one
quantity with no pin is listed as "parity unpinned" in ``closed_forms``.
"""

from . import attention, closed_forms, fp8, pool, transfer  # noqa: F401
