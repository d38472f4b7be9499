"""fp64 CPU oracle of the fused MXFP4 MoE expert layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The GPU library never calls it,
and it shares no code, tables or constants with the GPU library.

Everything here is plain NumPy in float64, written from the definitions on
the source pages:
  * the MoE dataflow (prepare map -> GEMM1 -> SiLU-and-mul -> GEMM2 ->
    shuffle-mul-sum) from "SGLang CUTLASS MoE" (structure diagram, sections
    1, 4 and 5);
  * the expert offset, the -1 slots and the virtual-expert bound
    kMaxV = E + T*topk/BlockN from "Generalizing the Kimi-K3.1 MXFP4 decode
    MoE kernel with a Shape template" (sections 1, 3 and 5);
  * the sigmoid shared-expert append from "SGLang MoE shared expert:
    fusing three kernels into one" (the append kernel, after the change);
  * the device-side Dense/Split GEMM2 choice from "FlashInfer device-side
    gating of the MoE GEMM2 path" (sections 1 and 2);
  * FP4 (E2M1) activations for the W4A4 variant from "SGLang CUTLASS MoE"
    (section 6), in the MX block format of the weights.

Functions whose result has no pin other than the oracle itself say
"parity unpinned" in their docstring.
"""
from .mx import (E2M1_MAGNITUDES, e2m1_decode, e8m0_decode, dequant_mxfp4,
                 quant_mxfp8, dequant_mxfp8, e4m3_decode, quant_mxfp4, pack_nibbles)
from .moe import (route_topk_softmax, shared_append, local_map, sort_align,
                  kmax_v, gate_word, dense_tiles, expert_glu, situ, reference_forward,
                  sampled_forward, GATE_TAU, DENSE_MT, bf16_bits_to_f64)

__all__ = [
    "E2M1_MAGNITUDES", "e2m1_decode", "e8m0_decode", "dequant_mxfp4", "quant_mxfp8",
    "quant_mxfp4", "pack_nibbles",
    "dequant_mxfp8", "e4m3_decode", "route_topk_softmax", "shared_append", "local_map",
    "sort_align", "kmax_v", "gate_word", "dense_tiles", "expert_glu", "situ", "reference_forward",
    "sampled_forward", "GATE_TAU", "DENSE_MT", "bf16_bits_to_f64",
]
