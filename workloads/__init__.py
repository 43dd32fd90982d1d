"""Seeded synthetic inputs for the multi-tenant LoRA linear layer.

This module serves both the GPU library's tests and benchmark and the CPU
oracle, so it holds none of the layer's arithmetic: it only draws random
values (numpy PCG64), rounds them to bf16 with torch's own conversion, and
builds the integer metadata (tenant indices, masks, ranks).

Shapes follow the layers the method is measured on ("EpiLoRA: Fusing Many
LoRA Adapters into Low-Precision GEMMs for Serving and RL", Evaluation,
Setup: Llama-3.1-8B and Qwen2.5-72B layer shapes; the adapters there are
random draws of ranks 16 to 128, because their shapes alone set the
kernels' speed) and the prefill-only
serving case ("PreFT: Prefill-only finetuning for efficient inference",
abstract: 512 adapters on a 70B-class model).

Value distributions: X ~ N(0, 1), W ~ N(0, 0.02), A ~ N(0, 1/sqrt(K)),
B ~ N(0, 0.01) (the second argument is the standard deviation); the LoRA
scaling is 2.0.  Every tensor has its own seed, derived from
(config, gemm, tensor, adapter), so a tensor can be drawn alone and adapters
no token references need not be drawn at all.
"""

from .configs import (  # noqa: F401
    GEMMS_8B,
    GEMMS_72B,
    SLICES_8B,
    SLICES_72B,
    GemmCase,
    Layer,
    bf16_bits,
    config,
    custom_layer,
)
