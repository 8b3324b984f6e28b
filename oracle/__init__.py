"""CPU oracle for the routed MoE layer served from an elastic expert cache.

TEST INFRASTRUCTURE.  Plain, slow, obviously-correct NumPy / pure-Python code
that states what the layer computes.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does.
It shares no code with the HIP library or its Python binding and imports
nothing from them.

Floating point is fp64 from the exact bf16 inputs, except the router logits,
whose fp32 summation order is part of the definition (see ``router``).
Integer decisions (top-k ids, permutation, cache hits/misses, q*, slots) are
exact integer arithmetic.

Citations used throughout:
  [FT]  the paper "FreeToken: Efficient Edge-Native MoE Serving with
        Bandwidth-Adaptive Execution" (arXiv 2608.16157), by section/equation.
  [AIN] the page "FreeToken: bandwidth-adaptive edge MoE serving"
        (ai-infrastructure.net), by section heading.
  [CN]  the Chinese translation of the paper on 10100.com, which carries the
        full body of Table 1.

Modules:
  router   logits, top-k, gates                      -- parity pinned
  ffn      SwiGLU expert FFN, sparse and dense layer -- parity pinned
  qstar    fetch fraction and the integer split q    -- parity pinned
  cache    two independent LRU residency simulators  -- parity pinned
  permute  stable grouping of (token, slot) pairs    -- parity pinned
  layer    decode / prefill layer composition        -- pinned through the above
  placement  Fig. 4b placement replay (LRU, hot set, static split) -- parity pinned
"""
