"""GPU parity of the decoder stack (layers + the final RMSNorm,
llama_stack_forward) against the oracle's model forward, and HIP-graph
replays of a captured stack forward against eager runs; also for stacks of
Qwen3-MoE-structured layers."""
import numpy as np
import pytest
import torch

import llama_decoder_layer_amd as lda
import oracle
import synth
from tests import stages
from tests.parity import (COS_MIN, compare, cosine, device_batch, device_qsl, moe_check_weights, moe_fix_routing,
                          np64, oracle_seqs, oracle_weights, run_oracle)

pytestmark = pytest.mark.gpu
DEV = "cuda"
MID = synth.ModelShape(1024, 8, 2, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")
# 8 query heads per KV head, one KV head: few query tiles, so long contexts split
MID8 = synth.ModelShape(1024, 8, 1, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")


def _stack_inputs(wl, layers):
    batch = synth.build_batch(wl)
    hidden, _ = synth.draw_activations(wl.model, batch.num_tokens, wl.index, DEV, residual=False)
    weights = [synth.draw_weights(wl.model, wl.index, l, DEV) for l in range(layers)]
    pools = [synth.build_kv_pool(wl, batch, l, DEV) for l in range(layers)]
    final = synth.draw_final_norm(wl.model, wl.index, DEV)
    return batch, hidden, weights, pools, final


def _final_norm_refs(h, r, final, eps):
    """(exact, bf16-storage) references of the final norm of the GPU's last
    (hidden, residual) pair: the storage oracle rounds the sum before the
    norm; neither rounds the output."""
    he, re_, w = np64(h), np64(r), np64(final)
    exact = oracle.rms_norm(he + re_, w, eps)
    rounded = oracle.rms_norm(oracle.bf16_round(he + re_), w, eps)
    return exact, rounded


def test_mid_stack_mixed_batch_vs_oracle():
    """Three layers and the final norm on a mixed batch.  The stack equals the
    chain of single-layer forwards plus the norm op bitwise; each layer is
    checked with the oracle fed that layer's GPU inputs, the final norm on
    the GPU's last pair, and the output end to end (cosine) against the
    oracle's own chain."""
    layers = 3
    mix = ((1, 700), (30, 0), (9, 40))
    wl = synth.Workload(50, "mid_stack3_mixed", MID, len(mix), 0, mix=mix)
    batch, hidden, weights, pools, final = _stack_inputs(wl, layers)
    pools0 = [(k.clone(), v.clone()) for k, v in pools]
    stack = lda.Stack(MID.config_dict(), weights, final)
    pos, bt, sl = device_batch(batch, DEV)
    qsl = device_qsl(batch, DEV)
    out = stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, query_start_loc=qsl)
    torch.cuda.synchronize()
    stack.close()
    cfg = MID.config_dict()
    # the same layers one at a time on fresh copies of the pools
    h, r, ins, outs, wss = hidden, None, [], [], []
    T, B = batch.num_tokens, batch.num_seqs
    for l in range(layers):
        kp, vp = pools0[l][0].clone(), pools0[l][1].clone()
        L = lda.Layer(cfg, weights[l])
        ws = L.alloc_workspace(T, B, batch.max_seq_len)
        ho, ro = L.forward(h, r, pos, kp, vp, bt, sl, batch.max_seq_len, workspace=ws, query_start_loc=qsl)
        torch.cuda.synchronize()
        wss.append(stages.workspace(L, ws, T, B, batch.max_seq_len))
        L.close()
        ins.append((h, r))
        outs.append((ho, ro))
        h, r = ho, ro
    for l in range(layers):
        ho, ro = outs[l]
        if not (torch.isfinite(ho.float()).all() and torch.isfinite(ro.float()).all()):
            raise AssertionError("chained layer %d: %s" % (l, stages.nan_report(wss[l], {"hidden_out": ho,
                                                                                        "residual_out": ro})))
    chained, _ = lda.add_rmsnorm(h, r, final, MID.rms_norm_eps, write_residual=False)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), chained.view(torch.int16))
    wn = [oracle_weights(w) for w in weights]
    seqs = [oracle_seqs(MID, batch, k0, v0) for k0, v0 in pools0]
    for l in range(layers):
        exact, rounded = run_oracle(MID, wn[l], ins[l][0], ins[l][1], batch, seqs[l])
        s1 = compare("hidden_out[%d]" % l, np64(outs[l][0]), exact["hidden_out"], rounded["hidden_out"])
        s2 = compare("residual_out[%d]" % l, np64(outs[l][1]), exact["residual_out"], rounded["residual_out"])
        print("layer", l, "hidden_out", s1, "residual_out", s2, flush=True)
    exact, rounded = _final_norm_refs(h, r, final, MID.rms_norm_eps)
    print("final norm", compare("stack_out", np64(out), exact, rounded), flush=True)
    posn = batch.positions.numpy().astype(np.int64)
    chain, _ = oracle.model_forward(cfg, wn, np64(final), np64(hidden), posn, seqs)
    cos = cosine(np64(out), chain)
    print("stack out vs the oracle's own chain: cos %.7f" % cos, flush=True)
    assert cos >= COS_MIN


def test_stack_graph_replays_match_eager():
    layers = 2
    wl = synth.Workload(51, "mid_stack2_decode_b8", MID, 8, 1, (5, 900))
    batch, hidden, weights, pools, final = _stack_inputs(wl, layers)
    stack = lda.Stack(MID.config_dict(), weights, final)
    pos, bt, sl = device_batch(batch, DEV)
    T, B = batch.num_tokens, batch.num_seqs
    ws = stack.alloc_workspace(T, B, batch.max_seq_len)
    side = torch.cuda.Stream()
    # eager reference on the side stream
    out_eager = torch.empty_like(hidden)
    stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=out_eager, workspace=ws, stream=side)
    side.synchronize()
    out = torch.zeros_like(hidden)
    graph = stack.capture(hidden, pos, pools, bt, sl, batch.max_seq_len, out, ws, side)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.launch(side)
        side.synchronize()
        assert torch.equal(out.view(torch.int16), out_eager.view(torch.int16)), "replay %d" % i
        # eager work between replays: an unrelated eager forward into another buffer
        scratch = torch.empty_like(hidden)
        stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=scratch, workspace=ws, stream=side)
        side.synchronize()
        assert torch.equal(scratch.view(torch.int16), out_eager.view(torch.int16))
    # the graph reads the input buffer's contents at launch time
    hidden.copy_(hidden.flip(0))
    torch.cuda.synchronize()
    ref2 = torch.empty_like(hidden)
    stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=ref2, workspace=ws, stream=side)
    side.synchronize()
    assert not torch.equal(ref2, out_eager)
    for i in range(2):
        graph.launch(side)
        side.synchronize()
        assert torch.equal(out.view(torch.int16), ref2.view(torch.int16)), "replay on new input %d" % i
    graph.close()
    stack.close()


def test_stack_graph_mixed_batch_split_attention_replays():
    # a mixed batch whose prefill tiles split their keys and whose decode rows
    # run on the decode kernel (row map, partition counts, combine), captured
    # once and replayed: every replay bit-identical to the eager forward
    layers = 2
    mix = ((1, 1500), (40, 1000), (1, 300), (3, 700))
    wl = synth.Workload(52, "mid8_stack2_mixed_split", MID8, len(mix), 0, mix=mix)
    batch, hidden, weights, pools, final = _stack_inputs(wl, layers)
    stack = lda.Stack(MID8.config_dict(), weights, final)
    pos, bt, sl = device_batch(batch, DEV)
    qsl = device_qsl(batch, DEV)
    T, B = batch.num_tokens, batch.num_seqs
    ws = stack.alloc_workspace(T, B, batch.max_seq_len)
    side = torch.cuda.Stream()
    out_eager = torch.empty_like(hidden)
    stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=out_eager, workspace=ws, stream=side,
                  query_start_loc=qsl)
    side.synchronize()
    out = torch.zeros_like(hidden)
    graph = stack.capture(hidden, pos, pools, bt, sl, batch.max_seq_len, out, ws, side, query_start_loc=qsl)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.launch(side)
        side.synchronize()
        assert torch.equal(out.view(torch.int16), out_eager.view(torch.int16)), "replay %d" % i
        scratch = torch.empty_like(hidden)
        stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=scratch, workspace=ws, stream=side,
                      query_start_loc=qsl)
        side.synchronize()
        assert torch.equal(scratch.view(torch.int16), out_eager.view(torch.int16))
    graph.close()
    stack.close()


def test_stack_graph_capture_with_debug_checks_on(monkeypatch):
    # LLAMA_DEBUG=1 makes an eager forward check its metadata and wait for the
    # answer; under capture the check is skipped (a capture cannot wait), so
    # capturing still works and the replays match the (checked) eager forward
    monkeypatch.setenv("LLAMA_DEBUG", "1")
    layers = 2
    wl = synth.Workload(53, "mid_stack2_decode_b4_debug", MID, 4, 1, (5, 300))
    batch, hidden, weights, pools, final = _stack_inputs(wl, layers)
    stack = lda.Stack(MID.config_dict(), weights, final)
    pos, bt, sl = device_batch(batch, DEV)
    T, B = batch.num_tokens, batch.num_seqs
    ws = stack.alloc_workspace(T, B, batch.max_seq_len)
    side = torch.cuda.Stream()
    out_eager = torch.empty_like(hidden)
    stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=out_eager, workspace=ws, stream=side)
    side.synchronize()
    out = torch.zeros_like(hidden)
    graph = stack.capture(hidden, pos, pools, bt, sl, batch.max_seq_len, out, ws, side)
    for i in range(2):
        out.zero_()
        torch.cuda.synchronize()
        graph.launch(side)
        side.synchronize()
        assert torch.equal(out.view(torch.int16), out_eager.view(torch.int16)), "replay %d" % i
    graph.close()
    stack.close()


def _moe_model():
    from tests.test_gpu_moe import MOE
    return MOE


def test_moe_stack_equals_chained_layers_and_oracle():
    """Three Qwen3-MoE-structured layers and the final norm: the stack is
    bitwise the chain of single-layer forwards plus the norm op.  Each layer
    is checked with the oracle fed that layer's GPU inputs (its routing
    validated, rows with a near-tie expert choice compared against the
    oracle's mixture over the GPU's experts), the final norm on the GPU's
    last pair, and the output end to end (cosine) against the oracle's own
    chain on the rows whose expert choices agree in every layer."""
    from tests.test_gpu_moe import _routing
    model = _moe_model()
    layers = 3
    wl = synth.Workload(52, "moe_stack3_decode_b24", model, 24, 1, (30, 500))
    batch, hidden, weights, pools, final = _stack_inputs(wl, layers)
    pools0 = [(k.clone(), v.clone()) for k, v in pools]
    cfg = model.config_dict()
    pos, bt, sl = device_batch(batch, DEV)
    T, B = batch.num_tokens, batch.num_seqs
    # chained single layers, keeping each layer's inputs, outputs and routing
    h, r, ins, outs, routing = hidden, None, [], [], []
    for l in range(layers):
        L = lda.Layer(cfg, weights[l])
        ws = L.alloc_workspace(T, B, batch.max_seq_len)
        ho, ro = L.forward(h, r, pos, pools[l][0], pools[l][1], bt, sl, batch.max_seq_len, workspace=ws)
        torch.cuda.synchronize()
        routing.append(_routing(L, ws, T, B, batch.max_seq_len))
        L.close()
        ins.append((h, r))
        outs.append((ho, ro))
        h, r = ho, ro
    chained, _ = lda.add_rmsnorm(h, r, final, model.rms_norm_eps, write_residual=False)
    for l in range(layers):  # the stack rewrites the same K/V slots
        pools[l][0].copy_(pools0[l][0])
        pools[l][1].copy_(pools0[l][1])
    stack = lda.Stack(cfg, weights, final)
    out = stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len)
    torch.cuda.synchronize()
    stack.close()
    assert torch.equal(out.view(torch.int16), chained.view(torch.int16))

    wn = [oracle_weights(w) for w in weights]
    seqs = [oracle_seqs(model, batch, k0, v0) for k0, v0 in pools0]
    posn = batch.positions.numpy().astype(np.int64)
    for l in range(layers):
        ids, wts, logits = routing[l]
        hin = np64(ins[l][0])
        rin = None if ins[l][1] is None else np64(ins[l][1])
        tr_e, tr_r = {}, {}
        exact = oracle.decoder_layer(cfg, wn[l], hin, rin, posn, seqs[l], trace=tr_e)
        rounded = oracle.decoder_layer(cfg, wn[l], hin, rin, posn, seqs[l], rnd=oracle.bf16_round, trace=tr_r)
        moe_check_weights(cfg, tr_r, ids, wts, logits)
        n_fix = moe_fix_routing(cfg, wn[l], tr_e, exact, ids)
        moe_fix_routing(cfg, wn[l], tr_r, rounded, ids, rnd=oracle.bf16_round)
        s1 = compare("hidden_out[%d]" % l, np64(outs[l][0]), exact["hidden_out"], rounded["hidden_out"])
        s2 = compare("residual_out[%d]" % l, np64(outs[l][1]), exact["residual_out"], rounded["residual_out"])
        print("layer", l, "near-tie rows", n_fix, "hidden_out", s1, "residual_out", s2, flush=True)
    exact, rounded = _final_norm_refs(h, r, final, model.rms_norm_eps)
    print("final norm", compare("moe_stack_out", np64(out), exact, rounded), flush=True)
    # end to end: the oracle's own chain, on rows routed alike in every layer
    keep = np.ones(T, dtype=bool)
    he, re_ = np64(hidden), None
    for l in range(layers):
        tr = {}
        o = oracle.decoder_layer(cfg, wn[l], he, re_, posn, seqs[l], trace=tr)
        for t in range(T):
            if set(int(e) for e in routing[l][0][t]) != set(int(e) for e in tr["topk_ids"][t]):
                keep[t] = False
        he, re_ = o["hidden_out"], o["residual_out"]
    chain, _ = oracle.fused_add_rms_norm(he, re_, np64(final), cfg["rms_norm_eps"])
    print("rows routed alike through the chain", int(keep.sum()), "of", T, flush=True)
    assert keep.sum() >= T // 2
    cos = cosine(np64(out)[keep], chain[keep])
    print("moe stack out vs the oracle's own chain: cos %.7f" % cos, flush=True)
    assert cos >= COS_MIN


def test_moe_stack_graph_replays_match_eager():
    model = _moe_model()
    wl = synth.Workload(53, "moe_stack2_decode_b16", model, 16, 1, (5, 700))
    batch, hidden, weights, pools, final = _stack_inputs(wl, 2)
    stack = lda.Stack(model.config_dict(), weights, final)
    pos, bt, sl = device_batch(batch, DEV)
    T, B = batch.num_tokens, batch.num_seqs
    ws = stack.alloc_workspace(T, B, batch.max_seq_len)
    side = torch.cuda.Stream()
    out_eager = torch.empty_like(hidden)
    stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=out_eager, workspace=ws, stream=side)
    side.synchronize()
    out = torch.zeros_like(hidden)
    graph = stack.capture(hidden, pos, pools, bt, sl, batch.max_seq_len, out, ws, side)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.launch(side)
        side.synchronize()
        assert torch.equal(out.view(torch.int16), out_eager.view(torch.int16)), "replay %d" % i
        scratch = torch.empty_like(hidden)
        stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, out=scratch, workspace=ws, stream=side)
        side.synchronize()
        assert torch.equal(scratch.view(torch.int16), out_eager.view(torch.int16))
    graph.close()
    stack.close()
