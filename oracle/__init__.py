"""CPU oracle for the direct-access split operators -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct reference of what the split operators compute,
written from the DAK paper ("DAK: Direct-Access-Enabled GPU Memory Offloading
with Optimal Efficiency for LLM Inference", Lin, Guo and Lin) and its Chinese
walkthrough (pinghaoyang.com.cn, "DAK 完全拆解"), in numpy fp64.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product package.  The two share only ``synth`` (seeded input
generation, no arithmetic of the method).

Modules:
  gemm        -- C = A.B with A split by tile-rows across two tiers (DAK §4.1)
  attention   -- exact decode attention with the KV cache split along the batch (DAK §5)
  cost_model  -- T_g, T_h, T = max(T_comp, T_g, T_h), EB, turning points (DAK §4.2.1)
  planner     -- global capacity ratio and the three-phase greedy per-op planner (DAK §4.2.2)
  brute       -- exhaustive search over per-op plans for tiny op sets (DAK App. A, eq. 1)
  schedule    -- host work-group count from wave alignment under a host-CU cap (DAK §4.1, §4.3.1)
  fp8         -- the split GEMM over FP8 (OCP E4M3) weights with per-row scales (BOOST §5 runs FP8 models)

Parity status: every function here is pinned by a ``-m "not gpu"`` test against
values the pages print, closed forms or brute force (see tests/test_oracle_*.py).
"""
from . import gemm, attention, cost_model, planner, brute, schedule  # noqa: F401
