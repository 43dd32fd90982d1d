"""CPU oracle for the multi-tenant LoRA linear layer on a low-precision base.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the layer computes.  Only the tests, the smoke check and
the benchmark's CPU-baseline leg may import it.  The GPU library never calls
it, and it imports nothing from the GPU package: the two share no code.

What it follows (page titles and sections of the method's description):

* "EpiLoRA: Fusing Many LoRA Adapters into Low-Precision GEMMs for Serving
  and RL", Background ("Why engines do not merge adapters", "The cost of the
  separate adapter path") and Design, section "Multi-adapter kernels"
  (K1 and K2, the decode path).
* "PreFT: Prefill-only finetuning for efficient inference", abstract and the
  caption of Figure 6 (the per-forward position mask).

The pages never spell out the number formats.  The readings used here (OCP
FP8 E4M3FN for "FP8", the NVFP4 block layout for the 4-bit weights, and the
fold of a 4-bit code with its block scale into one FP8 byte) are listed,
with their reasons, in the repository's design notes.

Precision: where a floating-point step decides an integer (a quantised code
or scale), it is taken in fp32, as the kernels take it.  Every sum of
products (the GEMM, the shrink, the expand) is taken in fp64.
"""

from .formats import (  # noqa: F401
    bf16_to_f32,
    f32_to_bf16,
    e4m3_decode_table,
    e4m3_decode,
    e4m3_encode,
    e2m1_decode_table,
    e2m1_encode,
    fold_table,
)
from .linear import (  # noqa: F401
    quant_rows_e4m3,
    quant_act,
    quant_weight_fp8,
    quant_weight_fp4,
    unpack_fp4,
    fold_decode_fp4,
    exact_decode_fp4,
    base_fp8,
    base_w8a16,
    base_fp4,
    active_rows,
    quant_adapter_fp8,
    adapter_values,
    shrink,
    expand,
    linear_lora,
    slice_bounds,
    linear_lora_sliced,
    rmsnorm,
    norm_quant_shrink,
)
