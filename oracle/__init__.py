"""CPU oracle for the quantized routed MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call, link or execute anything in this
package.  Only the test suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the GPU
path: it decodes the quantised packs, routes, sorts, multiplies and rounds
with its own NumPy / pure-Python code.

Two implementations live here:

* ``oracle.ref``   -- NumPy float64, vectorised; usable up to the full
  decode/prefill shapes (it dequantises only the experts a call touches).
* ``oracle.brute`` -- scalar pure Python for tiny inputs.  It decodes e2m1
  from the sign/exponent/mantissa bit fields instead of a table, sorts by
  trying every subset, and loops over every multiply-add, so that it pins
  ``oracle.ref`` independently.

Sources for what is computed (the pages only describe the layer in prose):

* the routed-expert kernel reads the weights of the activated experts only,
  block-sparse -- "antirez ds4: DeepSeek Metal inference" (ainews.cool),
  section "技术深度解析" (technical deep dive), which also gives 64 experts
  with top-2 routing and on-the-fly dequantisation;
* the routed-expert count is a run-time knob -- Anemll/ds4-ssd README,
  section "Experimental Pro Support" (``--moe-expert-topk``);
* MXFP4 routed experts -- Anemll/ds4-ssd README, section "Run SSD Sidecar
  Mode" (native MXFP4 package); e2m1 values and the e8m0 scale follow the
  OCP Microscaling Formats (MX) v1.0 specification;
* 2-bit asymmetric quantisation -- "DwarfStar 4 (ds4) | Mac Studio ...
  完整指南" (res.pawin.top), section "为什么 ds4 是 128GB Mac Studio 的最佳路径".
* the router must stay in full precision -- same guide, section "避坑指南".

Every reading taken where the pages are silent is listed in the docstring of
the function that takes it (and collected in the repository's design notes).
"""

from . import ref, brute  # noqa: F401
