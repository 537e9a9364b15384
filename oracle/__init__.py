"""FP64 CPU oracle for the routed-expert MoE FFN and its align-and-sort.

This package is TEST INFRASTRUCTURE. Only the test suite, the smoke entry
point and the benchmark's CPU-baseline leg may import it. The product path
(the HIP library and its Python binding) never imports, calls or links
anything here, and nothing here imports the product path: the two share no
kernels, helpers, tables or constants. Both sides read the same seeded inputs
from the separate ``workloads`` package, which holds none of the method's
arithmetic.

What is computed, and where it comes from:

* ``formats``   -- exact decoders for the stored number formats (E4M3FN, E2M1,
  E8M0, BF16) and the MX block quantiser used when the expert-centric path
  quantises activations.  The element encodings are the OCP ones; the pages
  only name the formats (warp-decode post, section on how the two kernels work:
  MXFP8 weights converted to FP32 on the fly; GC-MoE abstract: FP8/FP4).
* ``layer``     -- the MoE layer itself: y_t = sum_j w_tj * Wd_e (SiLU(Wg_e x_t) *
  Wu_e x_t), in float64, from identically dequantised weights (warp-decode post,
  sections on the traditional MoE path and on how the two kernels work), with
  exact activations (mode ``none``, the output-centric path) or with the
  expert-centric path's MX activations and BF16 slot outputs, h requantised
  with two terms (mode ``mxfp8``, what the grouped path computes) or one
  (mode ``mxfp8_single``, the plain reading of the pages).
* ``align_sort``-- the block-padded, expert-grouped ordering of (token, slot)
  entries (align-and-sort article, background section and the D-C-P section).
* ``router``    -- the router front-end: gating scores (+ bias) -> top-k ids and
  softmax weights over the selected scores (align-and-sort article, background
  and FasterTransformer sections).  ``workloads`` synthesises the routing
  *inputs* of the FFN path by its own recipe; the router kernel is checked
  only against this module.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against library routines, exhaustive enumerations, brute force and invariants.
No function is "parity unpinned".
"""

from . import formats, layer, align_sort, router  # noqa: F401
