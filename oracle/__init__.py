"""Float64 CPU oracle for the NVFP4 routed-MoE expert computation.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The HIP library never uses it and shares no code, tables or helpers with it.

What it computes follows these web pages (cited by page title and section):

* FlashInfer, "flashinfer.fused_moe.CudnnGroupedGemmNvfp4Config": the pipeline order
  (expert-sorted permutation, GEMM1, typed activation, GEMM2, finalize), the activation list
  (SwiGLU, GeGLU, GELU, ReLU, SiLU, Identity), 128-row segment
  padding, BF16 intermediate re-quantized to NVFP4 with a global scale of one, one global
  scale per expert, masking of non-local experts, the unfinalized output triple.
* Megatron-Core, "core.inference.moe.flashinfer_nvfp4": per-token NVFP4 x NVFP4 SwiGLU and
  squared-ReLU experts, the constants NVFP4_BLOCK_SIZE=16, FLOAT4_E2M1_MAX=6.0,
  FLOAT8_E4M3_MAX=448.0, one FP32 scale per token and per expert, "-1 rows contribute zero".
* FlashInfer, "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe": two E2M1 per byte with the
  even value in the low nibble, linear E4M3 scales per 16 values, the aligned routing plan
  (sorted_token_ids, expert_ids, num_tokens_post_padded), per-expert FP32 output scales,
  contributions added to the existing ``out`` in FP32.
* vLLM, "vllm.model_executor.layers.quantization.utils.flashinfer_utils":
  quantize_nvfp4_per_token_input returns one FP32 *decode* scale per token.
* FlashInfer, "flashinfer.fused_moe.FrostLowLatencyConfig": BF16 rounding of the activation
  output and of expert outputs; the FP4 weight-only mode (BF16 input, pre-activation and
  intermediate rounding); combine with every FP32 product and sum rounded separately, in slot
  order; expert
  ids outside the routed range are ignored together with their scores; packed routing scores
  keep their BF16 rounding (the packed word's layout is a reading stated in ``moe.unpack_routing``).

Where the pages are silent the reading taken is stated next to the code that takes it.

Every function here is pinned by ``tests/test_oracle_*.py`` against facts the pages and the
mathematics fix (format tables, exhaustive sweeps against a library float8 routine,
hand-derived golden values under ``tests/golden/``, exact rational brute force on tiny
inputs, invariants).  No function is "parity unpinned".
"""

from .formats import (  # noqa: F401
    E2M1_MAGNITUDES,
    FLOAT4_E2M1_MAX,
    FLOAT8_E4M3_MAX,
    NVFP4_BLOCK_SIZE,
    bf16_bits_to_f32,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    round_to_bf16,
    f64_to_bf16_bits,
)
from .mx import (  # noqa: F401
    MX_BLOCK_SIZE,
    dequantize_mxfp4,
    dequantize_mxfp8,
    e8m0_decode,
    mx_dot,
    quantize_mxfp4,
    quantize_mxfp8,
)
from .quant import SCALE_FIXED, SCALE_PER_GROUP, SCALE_PER_ROW, dequantize_nvfp4, quantize_nvfp4  # noqa: F401
from .moe import (  # noqa: F401
    ACT_GEGLU,
    ACT_GELU,
    ACT_IDENTITY,
    ACT_RELU,
    ACT_RELU2,
    ACT_SILU,
    ACT_SWIGLU,
    ACTS,
    is_gated,
    combine,
    dense_loop_moe,
    dense_loop_moe_mx,
    fused_moe_mx,
    expert_rows_forward_mx,
    expert_down_projection,
    expert_gate_up_projection,
    expert_rows_forward,
    expert_rows_forward_w16,
    fused_moe_nvfp4,
    fused_moe_w4a16,
    unpack_routing,
    moe_permute,
    moe_plan,
    plan_capacity,
    plan_violations,
    quantize_expert_rows,
    quantize_expert_weights,
    routing_violations,
    unquantized_moe_f64,
)
