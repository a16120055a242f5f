"""CPU oracle for the Llama decoder-layer forward (float64 numpy).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP library and imports nothing from it.
"""
from .layer import (STORAGE_POINTS, Seq, apply_rope, attend, bf16_round, decoder_layer,
                    decoder_stack, fused_add_rms_norm, linear, model_forward, rms_norm,
                    rope_frequencies, silu, silu_and_mul)
from .moe import (expert_ffn, head_rms_norm, mix_experts, router_logits, select_experts, softmax,
                  sparse_moe_block, topk_margin)

__all__ = ["STORAGE_POINTS", "Seq", "apply_rope", "attend", "bf16_round", "decoder_layer",
           "decoder_stack", "fused_add_rms_norm", "linear", "model_forward", "rms_norm", "rope_frequencies",
           "silu", "silu_and_mul", "expert_ffn", "head_rms_norm", "mix_experts", "router_logits",
           "select_experts", "softmax", "sparse_moe_block", "topk_margin"]
