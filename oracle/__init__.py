"""CPU oracle for the weight-only INT4/INT8 round-to-nearest MoE expert path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The library under
``weight_only_int4_rtn_amd`` never imports it, and it imports nothing from the
library: the two share no code.

Every function here is a plain, slow, readable statement of what the path
computes, written from the model-card pages this project follows:

* page "Nex-N2.5-mini Int4-Int8Mix", section Recipe: routed experts stored as
  symmetric INT4 with one min-max scale per group of 128, other projections as
  INT8 group 128, data-free round-to-nearest, fused expert banks split into
  per-expert 2-D ``[out, in]`` matrices, and a round-trip error band;
* page "Nex-N2.5-mini FP8 W8A8 with Calibrated FP8 KV Scales", section Artifact
  summary: 256 routed experts, 8 active per token;
* the same Int4-Int8Mix page, Recipe table: each routed expert is a
  gate_proj / up_proj / down_proj triple (a SwiGLU MLP); the router
  (``mlp.gate``) and the ``shared_expert_gate`` stay BF16.

* ``oracle.formats``: the FP8 E4M3 per-channel and MXFP4 expert formats of the
  pages "Nex-N2.5-mini-mixed-NVFP4-FP8" and "Nex-N2.5-mini-MXFP4-MxWave".

Where the pages leave a step open, the reading taken is stated at the function.
"""

from .rtn_moe import (  # noqa: F401
    GROUP,
    QMAX,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    rtn_quantize,
    pack_codes,
    unpack_codes,
    quantize_pack,
    dequantize,
    dequantize_as,
    route,
    router_logits,
    shared_gate,
    expert_ffn,
    moe_ffn,
    moe_layer,
    linear,
)

from . import formats  # noqa: E402,F401
