"""GPU parity of the Qwen3-MoE layer (llama_layer_forward with num_experts > 0
and qk_norm) against the oracle: decode batches on the weight-streaming expert
kernel (one and two 16-row passes per expert), prefill on the tiled expert
kernel (full and partly filled tiles), a mixed batch, the routing (router
logits, chosen experts, their weights), the KV cache, and bitwise-repeatable
output despite the atomics that group pairs by expert."""
import numpy as np
import pytest
import torch

import llama_decoder_layer_amd as lda
import oracle
import synth
from tests.parity import (compare, device_batch, device_qsl, moe_check_weights, moe_fix_routing, np64,
                          oracle_seqs, oracle_weights)
from tests import stages
from tests.test_gpu_layer import _check_kv, _check_metadata_unchanged

pytestmark = pytest.mark.gpu
DEV = "cuda"

# the Qwen3-MoE layer's structure at a small width: 8 query heads per KV head,
# head_dim 128, theta 1e7 without scaling, eps 1e-6, q/k norm, top-4 of 32
# experts (the 30B model: top-8 of 128)
MOE = synth.ModelShape(1024, 8, 1, 128, 2816, 1e-6, 1e7, None, 32768, "bf16",
                       num_experts=32, num_experts_per_tok=4, moe_intermediate_size=256,
                       norm_topk_prob=True, qk_norm=True)
# top-8 of 64, wider experts, GQA 4:1
MOE8 = synth.ModelShape(1024, 8, 2, 128, 2816, 1e-6, 1e7, None, 32768, "bf16",
                        num_experts=64, num_experts_per_tok=8, moe_intermediate_size=384,
                        norm_topk_prob=True, qk_norm=True)


def _routing(layer, ws, T, B, max_seq_len):
    ids = layer.workspace_tensor(ws, "topk_ids", T, B, max_seq_len).cpu().numpy()
    wts = np64(layer.workspace_tensor(ws, "topk_weights", T, B, max_seq_len))
    logits = np64(layer.workspace_tensor(ws, "router_logits", T, B, max_seq_len))
    return ids, wts, logits


def run_moe_layer(workload, ctx_lens=None, repeat=False, want=None, check_kv=None):
    """One MoE layer forward on the GPU and the oracle on the same tensors;
    checks outputs, routing and the KV cache.  Returns the GPU outputs."""
    model = workload.model
    batch = synth.build_batch(workload, ctx_lens)
    T, B = batch.num_tokens, batch.num_seqs
    print("case", workload.name, "T", T, "B", B, "ctx", batch.ctx_lens[:6], flush=True)
    hidden, residual = synth.draw_activations(model, T, workload.index, DEV, residual=not workload.residual_none)
    pos, bt, sl = device_batch(batch, DEV)
    qsl = device_qsl(batch, DEV)
    w = synth.draw_weights(model, workload.index, 0, DEV)
    kp, vp = synth.build_kv_pool(workload, batch, 0, DEV)
    kp0, vp0 = kp.clone(), vp.clone()
    meta0 = [t.clone() for t in (pos, bt, sl) + ((qsl,) if qsl is not None else ())]
    layer = lda.Layer(model.config_dict(), w)
    ws = layer.alloc_workspace(T, B, batch.max_seq_len)
    ho, ro = layer.forward(hidden, residual, pos, kp, vp, bt, sl, batch.max_seq_len, workspace=ws,
                           query_start_loc=qsl)
    torch.cuda.synchronize()
    _check_metadata_unchanged(meta0, pos, bt, sl, qsl)
    ids, wts, logits = _routing(layer, ws, T, B, batch.max_seq_len)
    qkv = layer.workspace_tensor(ws, "qkv", T, B, batch.max_seq_len).clone()
    table = layer.rope_table()
    wst = {n: t.clone() for n, t in stages.workspace(layer, ws, T, B, batch.max_seq_len).items()}
    if repeat:
        ho1, ro1 = ho.clone(), ro.clone()
        kp.copy_(kp0)
        vp.copy_(vp0)
        layer.forward(hidden, residual, pos, kp, vp, bt, sl, batch.max_seq_len, hidden_out=ho, residual_out=ro,
                      workspace=ws, query_start_loc=qsl)
        torch.cuda.synchronize()
        assert torch.equal(ho.view(torch.int16), ho1.view(torch.int16))
        assert torch.equal(ro.view(torch.int16), ro1.view(torch.int16))
    layer.close()

    cfg = model.config_dict()
    w_np = oracle_weights(w)
    seqs = oracle_seqs(model, batch, kp0, vp0)
    h = np64(hidden)
    r = None if residual is None else np64(residual)
    p = batch.positions.numpy().astype(np.int64)
    tr_e, tr_r = {}, {}
    exact = oracle.decoder_layer(cfg, w_np, h, r, p, seqs, want=want, trace=tr_e)
    rounded = oracle.decoder_layer(cfg, w_np, h, r, p, seqs, rnd=oracle.bf16_round, want=want, trace=tr_r)
    rows = exact["rows"]
    moe_check_weights(cfg, tr_r, ids[rows], wts[rows], logits[rows])
    n_fix = moe_fix_routing(cfg, w_np, tr_e, exact, ids[rows])
    n_fix_r = moe_fix_routing(cfg, w_np, tr_r, rounded, ids[rows], rnd=oracle.bf16_round)
    s1 = compare("hidden_out", np64(ho)[rows], exact["hidden_out"], rounded["hidden_out"])
    s2 = compare("residual_out", np64(ro)[rows], exact["residual_out"], rounded["residual_out"])
    print("rows with a near-tie expert choice", n_fix, n_fix_r, "hidden_out", s1, "residual_out", s2, flush=True)
    print(stages.summary(stages.check_stages(model, w_np, batch, hidden, residual, kp, vp, wst, ho, ro, rows)),
          flush=True)
    if (want is None) if check_kv is None else check_kv:
        _check_kv(model, batch, kp0, vp0, kp, vp, exact, rounded, qkv=qkv, table=table)
    return ho, ro, ids


def test_moe_decode_b24_streaming():
    run_moe_layer(synth.Workload(200, "moe_decode_b24", MOE, 24, 1, (60, 700)))


def test_moe_decode_b128_two_passes():
    # 128 tokens x 4 = 512 pairs on 32 experts: 16 per expert on average, so
    # the streaming kernel takes its two-pass (32-row) shape
    run_moe_layer(synth.Workload(201, "moe_decode_b128", MOE, 128, 1, (20, 300)))


def test_moe8_decode_b32():
    run_moe_layer(synth.Workload(202, "moe8_decode_b32", MOE8, 32, 1, (100, 900)))


def test_moe_prefill_2x1024_tiles():
    # 8192 pairs on 32 experts: 256 per expert on average, so full and partly
    # filled 256-row tiles both occur
    run_moe_layer(synth.Workload(203, "moe_prefill_2x1024", MOE, 2, 1024, 0), repeat=True)


def test_moe8_prefill_with_context():
    run_moe_layer(synth.Workload(204, "moe8_prefill_3x200_ctx", MOE8, 3, 200, (30, 400)))


def test_moe_mixed_chunk_and_decode():
    mix = tuple([(1, 300)] * 12 + [(150, 200)] + [(1, 40)] * 4)
    run_moe_layer(synth.Workload(205, "moe_mixed", MOE, len(mix), 0, mix=mix), repeat=True)


def test_moe_decode_repeat_bitwise():
    run_moe_layer(synth.Workload(206, "moe_decode_b64_repeat", MOE8, 64, 1, (10, 200)), repeat=True)


def test_moe_prefill_3x1000_chunked_grouping():
    # 12000 pairs: more than 8192, so the grouping by expert runs as count /
    # scan / scatter kernels over chunks of 4096 pairs (the last one ragged)
    run_moe_layer(synth.Workload(207, "moe_prefill_3x1000", MOE, 3, 1000, 0), repeat=True)


# 48 experts (not a multiple of 64: the top-k wave leaves lanes 48..63 empty),
# top-3 without renormalisation, head_dim 64 with 4 query heads per KV head
MOE48 = synth.ModelShape(512, 8, 2, 64, 1408, 1e-6, 1e7, None, 32768, "bf16",
                         num_experts=48, num_experts_per_tok=3, moe_intermediate_size=128,
                         norm_topk_prob=False, qk_norm=True)
# top-1 (every token's weight is exactly 1 after renormalising), no q/k norm
MOE1 = synth.ModelShape(512, 8, 2, 64, 1408, 1e-6, 1e7, None, 32768, "bf16",
                        num_experts=16, num_experts_per_tok=1, moe_intermediate_size=256,
                        norm_topk_prob=True, qk_norm=False)


def test_moe48_top3_unnormalised_decode_and_prefill():
    run_moe_layer(synth.Workload(208, "moe48_decode_b40", MOE48, 40, 1, (10, 300)))
    run_moe_layer(synth.Workload(209, "moe48_prefill_2x300", MOE48, 2, 300, (0, 64)))


def test_moe_top1_decode_and_prefill():
    _, _, ids = run_moe_layer(synth.Workload(210, "moe1_decode_b16", MOE1, 16, 1, (10, 300)))
    assert ids.shape == (16, 1)
    run_moe_layer(synth.Workload(211, "moe1_prefill_3x100", MOE1, 3, 100, 0))


# 128 experts with more than 128 tokens: the router runs on the tiled GEMM
# (split-K fp32 partials summed by the top-k kernel)
MOE128 = synth.ModelShape(512, 8, 1, 128, 1408, 1e-6, 1e7, None, 32768, "bf16",
                          num_experts=128, num_experts_per_tok=8, moe_intermediate_size=128,
                          norm_topk_prob=True, qk_norm=True)


def test_moe128_router_on_gemm_prefill():
    run_moe_layer(synth.Workload(212, "moe128_prefill_2x150", MOE128, 2, 150, (0, 40)))
    run_moe_layer(synth.Workload(213, "moe128_decode_b20", MOE128, 20, 1, (10, 200)))
