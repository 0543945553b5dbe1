"""CPU oracle for the routed-MoE decode/verify layer -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, float64 definition of what the layer
computes.  It is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``; nothing in the product path (the HIP
library and its Python binding) may import or call it, and it imports nothing
from the product path.  It shares no code with the HIP kernels: its own format
decoders, its own routing, its own union, its own FFN.

Sources (cited by page title and section, as the pages print them):

* "Function forward_moe" (rustdoc of ``spark_model::layers::glm5next_mlp::
  forward::forward_moe``): signature (x in, out out, ``rows``); the
  "amortize PARTIALLY" note (union of selected experts over verify rows);
  the "RETRACTED (2026-08-29)" note (top_k*rows <= 64 ids deduplicated in one
  block by a pairwise scan without a sort; the union sweep and the per-row
  path give byte-identical outputs); the "WIDENED (2026-08-31)" note
  (rows <= 8); the SHARED-expert note (shared expert runs once over all rows).
* ``metrale_model_layers/layers/moe/forward_token_major.rs``,
  ``MoeLayer::forward_token_major_decode``: batched router GEMM, batched top-k
  (softmax with ``norm_topk_prob`` or sigmoid with a correction bias and
  ``routed_scaling_factor``), gate+up, silu+down, weighted sum plus blend of
  the shared expert, NVFP4 experts addressed by pointer tables
  (packed codes, block scales, ``scale2`` values).
* ``metrale_model_layers/layers/moe/forward_ep.rs``,
  ``MoeLayer::forward_ep_dispatch``: the one-row router GEMV and
  ``moe_topk_softmax`` with ``norm_topk_prob``.
* NVFP4 element formats follow the public OCP specifications (OCP
  Microscaling Formats v1.0 for E2M1; OCP 8-bit Floating Point for E4M3FN);
  the pages name the format only.

Parity status of each function is stated in its module.  Parity unpinned:
the pages' own ``router_input`` transform (read as identity), the union
order (first occurrence in row-major slot order: a reading, not printed on
the pages), and the pages' kernels' internal rounding (not reproduced; the
oracle is the plain definition).
"""

from . import formats, route, union, ffn, layer  # noqa: F401
