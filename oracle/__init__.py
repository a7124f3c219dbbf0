"""Plain CPU oracle for the routed-MoE layer under expert offloading.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library under
``expert_offloaded_routed_amd/`` (no kernels, headers, helpers, tables or constants); the two
meet only in the seeded inputs of the ``synthetic`` package.

Everything here is written for obviousness, not speed: numpy float64 (library matmul as a
single step), pure-Python loops only where the method is a small integer algorithm.

Modules:
  mxfp4         -- E2M1 element / E8M0 scale decode (OCP Microscaling Formats v1.0)
  formats       -- bf16, block FP8 (E4M3 + 128 x 128 fp32 scales) and NVFP4 (E2M1 + E4M3
                   per 16 + fp32 matrix scale) decode, the other expert formats
  layer         -- router, softmax/top-k/renormalise, SwiGLU expert FFN, ordered combine,
                   route buckets
  cache_policy  -- per-layer slot cache: LRU / LFRU victim choice, bounded refills per step,
                   fixed-lag visibility

Parity pins (tests/test_oracle_*.py) tie each function to something other than itself; the
absolute outputs of the large workloads are otherwise pinned only through the definitions and
invariants (no page prints layer-level values).
"""
