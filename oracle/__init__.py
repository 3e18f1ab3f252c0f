"""CPU oracle for MoE token dispatch and combine.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package.  The only callers allowed are the test
suite under ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``.  The oracle shares no code with the HIP library: not
its kernels, headers, helpers, tables or constant generators.

It is deliberately plain and slow.  Every function states which passage of
the source pages it follows.  The pages are:

* "Low-Latency Mode API" (DeepEP-Ascend ``low_latency_dispatch`` /
  ``low_latency_combine``), sections Parameters, Return Values, Constraints.
* "DeepEP FP8 Dispatch and Combine Operations" (DeepEP article), sections
  "The Dispatch Stage", "Message Transmission via IBGDA", "The FP8 Combine
  Operation".
* "[feat] A5 deep fused moe" (sgl-kernel-npu pull request 661), section
  Testing (the fused-counts table).
* "EP dispatch with unfused MXFP8 quantization" (TransformerEngine pull
  request 3270), sections Description and Changes.
* "DeepEP topk_idx_t Custom Dtype Requirements", sections "Tensor
  Requirements and Constraints" and "Runtime Validation".

Where the pages are silent or garbled, each module states the reading it
takes.

Modules:

* ``codecs``   -- bf16, int8, OCP e4m3fn, OCP e2m1 and e8m0 element codecs.
* ``quant``    -- the seven per-row quantisation modes.
* ``layout``   -- expert histogram, exclusive scan, stable slot assignment.
* ``dispatch`` -- quantise each token once and copy it to each routed row.
* ``combine``  -- gather, dequantise, fp32 weighted sum in top-k order.
* ``backward`` -- combine's gradient with respect to the expert rows, as a
  reverse dispatch.
* ``moe``      -- the expert MLP between dispatch and combine (GMM1, SwiGLU,
  MXFP8 requant, GMM2).
* ``validate`` -- the argument rules the C ABI enforces before any launch.

Parity status of every function is listed in each module's header.
"""

from . import codecs, quant, layout, dispatch, combine, backward, validate, moe  # noqa: F401
from .layout import Layout  # noqa: F401

QUANT_MODES = ("none", "int8_token", "fp8_b128", "mxfp8", "mxfp4", "fp8_b128_pow2", "fp8_b128_ue8m0")
