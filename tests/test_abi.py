"""CPU-side checks of the C ABI: the library loads, exports exactly what the
header declares, and rejects bad configurations and arguments on the host
before touching a GPU."""
import ctypes
import os
import re

import pytest

import llama_decoder_layer_amd as lda
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"LLAMA_API\s+[\w\s\*]+?\b(llama_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert "llama_layer_forward" in declared and "llama_layer_create" in declared
    L = lda.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert declared == set(lda.EXPORTED)


def _cfg(**over):
    cfg = synth.LLAMA70B.config_dict()
    cfg.update(over)
    return cfg


def test_validate_70b_config_ok():
    assert lda.validate(_cfg()) == lda.Status.OK
    assert lda.validate(synth.TINY.config_dict(), lda.Dtype.FP32) == lda.Status.OK


@pytest.mark.parametrize("over,expect", [
    ({"hidden_act": "gelu"}, lda.Status.UNSUPPORTED),
    ({"attention_bias": True}, lda.Status.UNSUPPORTED),
    ({"mlp_bias": True}, lda.Status.UNSUPPORTED),
    ({"num_key_value_heads": 7}, lda.Status.INVALID_ARGUMENT),
    ({"head_dim": 96}, lda.Status.UNSUPPORTED),
    ({"rope_scaling": {"rope_type": "yarn", "factor": 4.0}}, lda.Status.UNSUPPORTED),
    ({"rope_scaling": dict(synth.LLAMA3_SCALING, high_freq_factor=1.0)}, lda.Status.INVALID_ARGUMENT),
    ({"rope_scaling": dict(synth.LLAMA3_SCALING, factor=0.5)}, lda.Status.INVALID_ARGUMENT),
    ({"kv_block_size": 32}, lda.Status.UNSUPPORTED),
    ({"hidden_size": 8000}, lda.Status.UNSUPPORTED),
    ({"intermediate_size": 1000}, lda.Status.UNSUPPORTED),
    ({"hidden_size": 0}, lda.Status.INVALID_ARGUMENT),
    ({"rms_norm_eps": 0.0}, lda.Status.INVALID_ARGUMENT),
    ({"rope_theta": 1.0}, lda.Status.INVALID_ARGUMENT),
    ({"num_attention_heads": 64, "num_key_value_heads": 2}, lda.Status.UNSUPPORTED),  # 32 per group
])
def test_validate_rejects(over, expect):
    assert lda.validate(_cfg(**over)) == expect
    if expect != lda.Status.OK:
        assert lda.lib().llama_layer_last_error()


def test_validate_null_and_bad_dtype():
    L = lda.lib()
    assert L.llama_layer_config_validate(None) == lda.Status.INVALID_ARGUMENT
    c = lda.make_config(_cfg(), lda.Dtype.BF16)
    c.dtype = 7
    assert L.llama_layer_config_validate(ctypes.byref(c)) == lda.Status.INVALID_ARGUMENT
    c = lda.make_config(_cfg(), lda.Dtype.BF16)
    c.hidden_act = None
    assert L.llama_layer_config_validate(ctypes.byref(c)) == lda.Status.UNSUPPORTED
    assert b"silu" in L.llama_layer_last_error()


def test_host_argument_errors_need_no_gpu():
    L = lda.lib()
    # NULL layer / NULL pointers are rejected before any HIP call
    assert L.llama_layer_forward(None, None, None, None, 1, None, None, 1, None, None, 1, 1, None, None, None,
                                 None) == lda.Status.INVALID_ARGUMENT
    assert L.llama_layer_workspace_bytes(None, 1, 1, 1) == 0
    assert L.llama_op_linear(0, None, None, 1, 1, 1, 0, None, None) == lda.Status.INVALID_ARGUMENT
    fake = ctypes.c_void_p(1 << 20)
    # bf16 shape rules
    assert L.llama_op_linear(0, fake, fake, 4, 128, 100, 0, fake, None) == lda.Status.INVALID_ARGUMENT
    assert L.llama_op_linear(0, fake, fake, 4, 100, 128, 0, fake, None) == lda.Status.INVALID_ARGUMENT
    assert L.llama_op_linear(0, fake, fake, 4, 128, 128, 5, fake, None) == lda.Status.INVALID_ARGUMENT
    # misaligned pointer
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L.llama_op_linear(0, odd, fake, 4, 128, 128, 0, fake, None) == lda.Status.INVALID_ARGUMENT
    assert L.llama_op_add_rmsnorm(0, fake, None, fake, 1e-5, 4, 100, fake, None, None) == lda.Status.INVALID_ARGUMENT
    assert L.llama_op_add_rmsnorm(0, fake, fake, fake, 1e-5, 4, 128, fake, None, None) == lda.Status.INVALID_ARGUMENT
    assert L.llama_op_reorder_gate_up(fake, 24, 128, fake, None) == lda.Status.INVALID_ARGUMENT
    assert L.llama_op_reorder_gate_up(fake, 32, 128, fake, None) == lda.Status.INVALID_ARGUMENT  # aliasing
    # the stack and its graphs
    cfg = lda.make_config(synth.LLAMA70B.config_dict(), lda.Dtype.BF16)
    out = ctypes.c_void_p()
    w = (lda.Weights * 1)()
    assert L.llama_stack_create(ctypes.byref(cfg), 0, w, fake, None, ctypes.byref(out)) == lda.Status.INVALID_ARGUMENT
    assert b"num_layers" in L.llama_layer_last_error()
    assert L.llama_stack_create(ctypes.byref(cfg), 1, None, fake, None, ctypes.byref(out)) == lda.Status.INVALID_ARGUMENT
    assert L.llama_stack_workspace_bytes(None, 1, 1, 1) == 0
    assert L.llama_stack_forward(None, fake, fake, 1, None, fake, 1, fake, None, 1, 1, fake, fake,
                                 None) == lda.Status.INVALID_ARGUMENT
    g = ctypes.c_void_p()
    assert L.llama_stack_graph_create(None, fake, fake, 1, None, fake, 1, fake, None, 1, 1, fake, fake, fake,
                                      ctypes.byref(g)) == lda.Status.INVALID_ARGUMENT
    assert L.llama_graph_launch(None, None) == lda.Status.INVALID_ARGUMENT


def _moe_cfg(**over):
    cfg = synth.QWEN3MOE.config_dict()
    cfg.update(over)
    return cfg


def test_validate_qwen3_moe_config_ok():
    assert lda.validate(_moe_cfg()) == lda.Status.OK
    c = lda.make_config(_moe_cfg(), lda.Dtype.BF16)
    assert (c.num_experts, c.num_experts_per_tok, c.moe_intermediate_size, c.norm_topk_prob, c.qk_norm) == \
        (128, 8, 768, 1, 1)


@pytest.mark.parametrize("over,dtype,expect", [
    ({}, lda.Dtype.FP32, lda.Status.UNSUPPORTED),                       # MoE is bf16 only
    ({"num_experts": 100}, lda.Dtype.BF16, lda.Status.UNSUPPORTED),     # not a multiple of 16
    ({"num_experts": 512}, lda.Dtype.BF16, lda.Status.UNSUPPORTED),
    ({"num_experts_per_tok": 0}, lda.Dtype.BF16, lda.Status.INVALID_ARGUMENT),
    ({"num_experts": 16, "num_experts_per_tok": 17}, lda.Dtype.BF16, lda.Status.INVALID_ARGUMENT),
    ({"moe_intermediate_size": 200}, lda.Dtype.BF16, lda.Status.UNSUPPORTED),
    ({"hidden_size": 1152}, lda.Dtype.BF16, lda.Status.UNSUPPORTED),    # % 128 but not % 256
    ({"num_experts": -1}, lda.Dtype.BF16, lda.Status.INVALID_ARGUMENT),
])
def test_validate_rejects_moe(over, dtype, expect):
    assert lda.validate(_moe_cfg(**over), dtype) == expect
    assert lda.lib().llama_layer_last_error()


def test_create_needs_expert_and_norm_weights():
    L = lda.lib()
    fake = ctypes.c_void_p(1 << 20)
    cfg = lda.make_config(_moe_cfg(), lda.Dtype.BF16)
    w = lda.Weights()
    for n in ("input_layernorm", "qkv_proj", "o_proj", "post_attention_layernorm", "q_norm", "k_norm"):
        setattr(w, n, fake.value)
    out = ctypes.c_void_p()
    # no router / expert weights
    assert L.llama_layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out)) == \
        lda.Status.INVALID_ARGUMENT
    assert b"expert" in L.llama_layer_last_error()
    for n in ("router", "experts_gate_up", "experts_down"):
        setattr(w, n, fake.value)
    w.q_norm = None
    assert L.llama_layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(out)) == \
        lda.Status.INVALID_ARGUMENT
    assert b"qk_norm" in L.llama_layer_last_error()
