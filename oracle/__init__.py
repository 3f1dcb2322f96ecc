"""CPU oracle for one MoE layer's forward pass -- TEST INFRASTRUCTURE ONLY.

Plain NumPy, written from the source pages, deliberately slow and direct.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library and never
imports it; the only shared module is ``workloads`` (seeded input generation,
none of the layer's arithmetic).

Sources, cited by page title and section:

* [FT-zh]  "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
  Execution", Chinese digest (paper.rainbus.top), sections Core method,
  Method steps, Technical novelty.
* [FT-en]  the same paper's simplified English reader (paperglide.net),
  sections System Architecture, Semantic-Aware Expert Caching, Elastic Memory
  Management, Figure 2.
* [Edge0]  "The other half of the memory wall: serving a 35B MoE model from SSD
  with trained route prediction" (translated, bittide.aicompass.dev),
  sections 2 (MoE routing, Quantization) and 3.1 (Problem, Executor paths,
  Math contract).

Modules:

* ``formats`` -- int4 affine group-64 and MXFP4 dequantisation of an expert blob.
* ``route``   -- router logits, softmax-top-k and sigmoid-group routing.
* ``cache``   -- dedup, hit/miss classification, miss split, K-victim LRU,
  slot update and cache rebuild (the integer path, as a simulator).
* ``lru_reference`` -- an independent textbook ordered-dict LRU used to pin
  ``cache``.
* ``ffn``     -- gathered expert SwiGLU over dequantised weights, the weighted
  combine, and the prefill permutation.

Floating point runs in float64 by default (``dtype`` selects float32, the
precision the baseline timing uses).  Every routing decision that floating
point settles is taken exactly as the method states it: expert ranking on the
float32 logit, group ranking on float64 sigmoid sums.
"""
