"""GPU parity of the decoder stack (layers + the final RMSNorm,
llama_stack_forward) against the oracle's model forward, and HIP-graph
replays of a captured stack forward against eager runs."""
import numpy as np
import pytest
import torch

import llama_decoder_layer_amd as lda
import oracle
import synth
from tests.parity import compare, device_batch, device_qsl, np64, oracle_seqs, oracle_weights

pytestmark = pytest.mark.gpu
DEV = "cuda"
MID = synth.ModelShape(1024, 8, 2, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")


def _stack_inputs(wl, layers):
    batch = synth.build_batch(wl)
    hidden, _ = synth.draw_activations(wl.model, batch.num_tokens, wl.index, DEV, residual=False)
    weights = [synth.draw_weights(wl.model, wl.index, l, DEV) for l in range(layers)]
    pools = [synth.build_kv_pool(wl, batch, l, DEV) for l in range(layers)]
    final = synth.draw_final_norm(wl.model, wl.index, DEV)
    return batch, hidden, weights, pools, final


def test_mid_stack_mixed_batch_vs_oracle():
    layers = 3
    mix = ((1, 700), (30, 0), (9, 40))
    wl = synth.Workload(50, "mid_stack3_mixed", MID, len(mix), 0, mix=mix)
    batch, hidden, weights, pools, final = _stack_inputs(wl, layers)
    pools0 = [(k.clone(), v.clone()) for k, v in pools]
    stack = lda.Stack(MID.config_dict(), weights, final)
    pos, bt, sl = device_batch(batch, DEV)
    out = stack.forward(hidden, pos, pools, bt, sl, batch.max_seq_len, query_start_loc=device_qsl(batch, DEV))
    torch.cuda.synchronize()
    stack.close()
    cfg = MID.config_dict()
    wn = [oracle_weights(w) for w in weights]
    seqs = [oracle_seqs(MID, batch, k0, v0) for k0, v0 in pools0]
    posn = batch.positions.numpy().astype(np.int64)
    exact, _ = oracle.model_forward(cfg, wn, np64(final), np64(hidden), posn, seqs)
    rounded, _ = oracle.model_forward(cfg, wn, np64(final), np64(hidden), posn, seqs, rnd=oracle.bf16_round)
    s = compare("stack_out", np64(out), exact, oracle.bf16_round(rounded), "bf16", depth=layers + 1)
    print("stack out", s, flush=True)


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
