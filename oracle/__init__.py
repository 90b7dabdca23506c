"""CPU oracle of the Hadamard-rotated 3-bit KV cache.

TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  It shares no code with the HIP
library (``decode_attention_okv_amd``) and the library never imports it.

Two modes:

* the *bit specification* of the write path in float32 (elementwise NumPy
  float32 operations only, every operation rounded to nearest-even), which the
  GPU must reproduce bit for bit: rotation, block scales, codes, packing;
* the *mathematics* of the read path in float64: dequantise the rotated cache,
  softmax(q1 K^T / sqrt(d)) V with q1 = U q, then rotate back with U^T.

Every function cites the passage of the pages it follows.  The pages are
"Orthogonally mixed 3-bit KV cache" (synthcore idea 1973; below: "the idea
card"), "Orthogonal Invariance in Activation Space: Fast Walsh-Hadamard
Transforms for KV Quantization" (below: "the OIQ report") and "Hardware-Fused
Fast Hadamard Transforms Enable Lossless 3-Bit KV-Cache Compression at 128K
Context Without Perplexity Drift" (below: "the news item").
"""
from .okv_ref import *  # noqa: F401,F403
from .okv_ref import __all__ as _ref_all
from .okv_calib import *  # noqa: F401,F403
from .okv_calib import __all__ as _calib_all

__all__ = list(_ref_all) + list(_calib_all)
