"""CPU oracles for the LoRA SwiGLU MLP, the fused LoRA linear, the RMSNorm in
front of the MLP and the grouped (MoE) MLP (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. The HIP product path never does.
"""
from .lora_mlp_oracle import (ADAPTER_KEYS, WEIGHT_KEYS, backward, base_mlp_rows,  # noqa: F401
                              bf16_round, bruteforce, dequant_int4, dequant_int4_bits,
                              flops, forward, forward_backward, merged_reference,
                              sigmoid, silu, unpack_int4)
from . import lora_linear_oracle as linear  # noqa: F401,E402  (the fused LoRA linear)
from . import rmsnorm_oracle as rmsnorm  # noqa: F401,E402  (RMSNorm, and RMSNorm then the MLP)
from . import moe_oracle as moe  # noqa: F401,E402  (one LoRA MLP per expert over grouped rows)
