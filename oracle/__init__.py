"""CPU oracle for the small-M NVFP4 W4A4 decode linear.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table or
constant generator with the HIP library under ``nvfp4_decode_linear_amd/``.

Subject: "ReSET: Accurate Latency-Critical NVFP4 Reasoning via Step-Aware
Temperature Scaling" (arXiv 2606.13233).  The GitHub README's section "Core
components", item 2 (``kernels/`` -- nvfp4r) states the problem: a small-M
(M <= 8) NVFP4 W4A4 decode linear that streams FP4 weights once and reuses
each loaded weight for every activation row.  The pages name NVFP4 but never
define it; the format follows the public NVFP4 description (E2M1 elements, one
E4M3 scale per 16 consecutive elements, one FP32 scale per tensor) with the
element encodings of the OCP Microscaling (MX) v1.0 specification, section
5.3.3 (FP4 E2M1), and the OCP 8-bit Floating Point specification (OFP8) v1.0,
E4M3 ("FN": no infinities, a single NaN mantissa pattern).

Parity status per function (see each docstring for its pins):
  e2m1_decode, e4m3_decode, e2m1_encode, e4m3_encode  pinned (exhaustive,
      library cast, brute force, spec tables under tests/golden/)
  global_scale, quantize_blocks, quantize, dequantize pinned (invariants,
      metamorphic relations, closed forms)
  linear_ref, linear_exact, tolerance_bound           pinned (Fraction-exact
      sums, unit-scale integer closed form)
  rms_norm_rows, silu_mul                             pinned (torch CPU library
      routines in float64)
  reset.token_entropy                                 pinned (closed forms,
      scipy's entropy of scipy's softmax, invariances)
  reset.step_update, reset.temperature                parity unpinned (the
      pages name the step-aware temperature and its hyper-parameters t_low and
      tau0 but give no formula; the module states the reading used)
  reset.scale_logits                                  one binary32 division
"""

from .nvfp4 import (  # noqa: F401
    BLOCK,
    E2M1_MAX,
    E4M3_MAX,
    NVFP4Tensor,
    dequantize,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    global_scale,
    linear_exact,
    linear_ref,
    pack_nibbles,
    quantize,
    quantize_blocks,
    tolerance_bound,
    unpack_nibbles,
)
from . import reset  # noqa: F401
from .stack import rms_norm_rows, silu_mul  # noqa: F401
