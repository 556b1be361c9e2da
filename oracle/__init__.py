"""Oracle for the BasisKV decode hot path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, float64 CPU statement of what the decode path
computes, written from "BasisKV: Value Latents for Communication and Key
Routing" (arXiv 2611.02583): its abstract, Figure 1's caption, the appendix
Table 4 (per-token state and read widths) and the Table 9 / Table 10 captions
(paged routing).  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its Python binding) never imports, calls or links anything here,
and nothing here imports the product path: the two share no code.

Modules
  basiskv_ref  numpy float64 implementation of every step (compress, route,
               select, attend, reconstruct, one decode step).
  brute        pure-Python loops for tiny inputs, using a different evaluation
               order (projected queries) and an exhaustive subset search, as an
               independent second statement for the pins in tests/.

Pins (tests/test_oracle.py) tie every function to something other than
itself: brute force and exhaustive enumeration on tiny inputs, the
closed form "predicted key == exact key" when the factors are exact, torch's
scaled_dot_product_attention for the k = all-pages case, numpy's stable
argsort for selection, exact recovery of the latent and residual by the
encoders, and the latent/reconstruction identity.  No function is left
"parity unpinned".
"""

from .basiskv_ref import (  # noqa: F401
    storage_to_f64,
    round_to_storage,
    compress_tokens,
    predicted_keys,
    route_page_scores,
    select_pages,
    attend_group,
    reconstruct,
    decode_step,
)
