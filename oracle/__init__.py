"""CPU oracle for the AuraFlow transformer forward and the flow-matching Euler + CFG update.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition that the GPU kernels are checked against. Only the test suite, the
smoke check and the bench's CPU-baseline leg may import it; the product path
(the C-ABI library and its Python binding) never does, and shares no code,
table or constant generator with it.

Numerics: numpy, float32 by default, float64 when ``dtype=np.float64`` is passed
(used to check the float32 oracle against itself). Library primitives used as
steps: matrix products (``@``), ``exp``, ``cos``/``sin``.

Sources (the web pages this follows), cited by tag throughout:
  [PIPE]  "Diffusers 中 AuraFlow 管线实战：从 bitsandbytes 量化到 torch.compile 加速"
  [DOCS]  "AuraFlow" — Diffusers v0.43.0 pipeline documentation (zh), same page in ko
  [TRANS] "Diffusers 中的 AuraFlowTransformer2DModel：架构解析与源码级使用指南"
  [DEEP]  "【深度拆解】AuraFlow从基座到技术实现：开源文生图新范式"

The pipeline's text encoder (UMT5, a random-weight workload) is in oracle/umt5.py.

Parity status. Every function is pinned by the CPU tests (tests/test_oracle_*.py)
against closed forms, invariants, brute force on tiny inputs or values the pages
print. The pages print no worked numeric example of a forward pass, so agreement
with the original trained model's numerics (beyond the readings listed in the
design notes) is not established; each reading is a self-consistent definition.
"""
from .spec import (AuraFlowConfig, find_multiple, weight_specs, count_parameters,
                   TINY, BLOCK_PAIR, FULL)
from .numerics import round_bf16, round_e4m3, mxfp8_qdq
from .transformer import (layer_norm, modulate, timestep_embedding, timestep_mlp,
                          pe_crop_indices, patchify, unpatchify, patch_embed,
                          attention, attention_bf16_operands, feed_forward, joint_block, single_block,
                          pre_final, embed, forward, Weights, mx_block)
from .sampling import sigma_schedule, cfg_combine, euler_step, cfg_euler_step

__all__ = [
    "AuraFlowConfig", "find_multiple", "weight_specs", "count_parameters",
    "TINY", "BLOCK_PAIR", "FULL", "round_bf16", "round_e4m3", "mxfp8_qdq", "mx_block",
    "layer_norm", "modulate", "timestep_embedding", "timestep_mlp", "pe_crop_indices",
    "patchify", "unpatchify", "patch_embed", "attention", "attention_bf16_operands", "feed_forward", "joint_block",
    "single_block", "pre_final", "embed", "forward", "Weights",
    "sigma_schedule", "cfg_combine", "euler_step", "cfg_euler_step",
]
