"""CPU reference ("oracle") for the routed-expert MoE layer hot path.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain, obviously correct
reference that the HIP library is checked against. Only the test suite, the
smoke check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it. The product path (the ``libsmoe`` HIP
library and its Python binding) never imports it and shares no code,
header, table or helper with it; the two meet only in the seeded input
generators of the ``workload`` package, which hold none of the layer's
arithmetic.

Precision: floating point is float64 except where a float decides an
integer result (the router logits that pick the top-k experts), which is
computed in float32 in a stated summation order that the GPU reproduces.
Where the pages fix a 16-bit format (fp16 activations between the expert
projections, fp16 layer output), the value is rounded to fp16 at that point.

Parity status of each function (pinned = checked in ``tests/`` against
something other than itself):
  router_logits_f32      pinned (float64 dot within the fp32 error bound;
                         exact small-integer cases; bias additivity)
  topk_experts           pinned (brute-force full sort; ties; k = E)
  routing_weights        pinned (sums to 1 over all experts; closed form)
  shared_gate            pinned (closed form on hand-built inputs)
  align_by_expert        pinned (sorted() with a (expert, slot) key;
                         invariants; per-expert slot order)
  dequant_int4           pinned (quantiser round trip within half a step;
                         hand-packed words)
  swiglu / routed FFN    pinned (dense float64 MLP written inline in the
                         test; exact small-integer case; token-wise vs
                         expert-wise equivalence)
  combine                pinned (k=1, w=1 identity; linearity)
  elb_accumulate/topm    pinned (bincount; sum of counts; split-call
                         additivity; brute-force ranking)
  shared_ffn             pinned (hand-worked layer: gate and up rows give
                         different results when swapped)
  moe_layer              pinned (a whole layer worked by hand, both passes,
                         tests/golden/layer_handworked.json; token-by-token
                         composition of the pinned pieces with bias, gated
                         shared experts and both passes; planted wiring
                         mistakes -- swapped shared gate/up, dropped gate,
                         renormalised weights, INT4 weights in the target
                         pass, dropped bias, dropped shared term -- each
                         fail these pins)
  layer outputs vs the pages: the pages print no worked numeric example of
                         a layer, so the pins above are hand-worked and
                         structural rather than the pages' own numbers.
"""

from .moe import (  # noqa: F401
    align_by_expert,
    combine,
    dequant_int4,
    elb_accumulate,
    elb_topm,
    moe_layer,
    routed_ffn_expertwise,
    routed_ffn_tokenwise,
    router_logits_f32,
    routing_weights,
    shared_ffn,
    shared_gate,
    swiglu,
    topk_experts,
)
