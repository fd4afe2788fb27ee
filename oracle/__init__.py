"""CPU oracle for the Inkling 2 Small routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  This package is the correctness authority that the
GPU path is compared against.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it;
the product library never calls into it and shares no code, tables or
constants with it.

It is deliberately plain and slow: numpy, float64 accumulation, one step per
definition, no blocking or fusion beyond what the definitions state.

Sources of the definitions (the pages are the four web pages on Inkling 2
Small; "p2" is the SGLang cookbook page, "p3" the TokenSpeed blog, "p4" the
Miles docs page, "p1" the SGLang blog):

* Layer shape: 384 routed experts, top-8, no shared experts, capped SwiGLU,
  hidden 4608 -- p3 "What's new in Inkling 2 Small" table; p4 section 1
  (sigmoid-routed MoE, soft-capped SwiGLU) and section 2 (hidden 4608,
  moe_ffn_hidden_size 2304).
* Router: sigmoid scores, additive bias, top-k fused -- p1 "Performance"
  (kernel fusion bullet).
* Expert formats: NVFP4 experts in layers 0-39, MXFP8 in 40-47 -- p2 section
  2 "Checkpoints"; p3 table "Checkpoint" row.  The element and block
  conventions (E2M1 / E4M3 / E8M0, NVFP4 = E2M1 + E4M3 per 16 + fp32 tensor
  scale, MXFP8 = E4M3 + E8M0 per 32) are the public OCP-MX and NVFP4
  conventions; the block sizes are pinned by the checkpoint sizes printed on
  p2 section 2 "Checkpoints" (see tests/test_oracle_pages.py).
* Activation quantization W4A4 / W8A8 -- p4 section 5.3; the NVFP4
  activation scale spans each expert's full input width -- p2 section 2
  "Parallelism".
* Dispatch / both expert GEMMs / capped SwiGLU / combine as the stages of
  one MoE forward -- p2 section 2 "MegaMoE".

Readings taken where the pages are silent are listed in formats.py and
layer.py next to the code that takes them.

Parity status: every function here is pinned by tests under tests/ marked
"not gpu" (brute force, library routines, closed forms, invariants, the
pages' printed sizes).  Parity to the real Inkling weights is unpinned: the
pages print no worked numeric example of the layer.
"""
from .formats import (  # noqa: F401
    E2M1_MAG, E4M3_MAG, e2m1_encode, e2m1_decode, e4m3_encode, e4m3_decode,
    e8m0_decode, bf16_round_f64, bf16_bits_to_f32,
    quantize_mxfp8, dequantize_mxfp8, quantize_nvfp4, dequantize_nvfp4, nvfp4_global_scale,
    pack_nibbles, unpack_nibbles,
)
from .layer import (  # noqa: F401
    OracleConfig, route, dispatch, expert_forward, expert_gate_up, expert_down, moe_layer, combine, act_scale,
    quantize_expert_weights, dequantize_expert, cap_swiglu,
)
