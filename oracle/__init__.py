"""CPU oracle for the paged FP8-e4m3 KV-cache decode step.

This package is TEST INFRASTRUCTURE. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (the HIP library and its Python binding) never imports, links
or calls anything here, and nothing here imports the product path.

It is a plain, slow and obviously correct statement of what the decode step
computes, in float64 numpy:

* ``e4m3``  -- the OCP FP8 E4M3 format: decode table from the bit layout, a
  nearest-code encoder with round-half-to-even and saturation, and a second,
  independent bit-level encoder used only to cross-check the first.
* ``paged`` -- the three operations of the step as the pages state them:
  the batched page-tag check, quantize-on-append into pool pages, and decode
  attention over the pages with dequantize-on-read and a plain softmax.
* ``ingest`` -- the prefill handoff into the decode cache: per-KV-head amax
  and scale calibration, and the page-by-page write of whole prompts.
* ``weights`` -- weight-only quantized decode GEMV: INT4 and FP8 e4m3
  weights with per-(row, 128-input group) scales, and the float64 product.

The pages this follows are the five web reports of Cloudflare's FP8 KV-cache /
page-tag post (remio.ai it/pt/ko, iitog.ru, manulx.blog). Each function names
the page and section it follows.
"""

from . import e4m3, ingest, paged, weights  # noqa: F401
