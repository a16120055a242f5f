"""The forward entry point that allocates nothing (llama_layer_forward_noalloc,
for callers that cannot allocate) against llama_layer_forward: bit-identical
outputs and KV-cache writes on two calls in a row on one layer, the second
with a smaller batch than the first (the scratch keeps the first call's
contents), and a call that would need more than the scratch holds rejected
with nothing written."""
import pytest
import torch

import llama_decoder_layer_amd as lda
import synth
from tests.parity import device_batch, device_qsl

pytestmark = pytest.mark.gpu
DEV = "cuda"
MID = synth.ModelShape(1024, 8, 2, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")
SCRATCH_BYTES = 64 << 20


def _both(layer, wl, ctx=None):
    """One batch through both entry points on identical copies of the cache."""
    batch = synth.build_batch(wl, ctx)
    T, B = batch.num_tokens, batch.num_seqs
    print("case", wl.name, "T", T, "B", B, "workspace bytes", layer.workspace_bytes(T, B, batch.max_seq_len), flush=True)
    assert layer.workspace_bytes(T, B, batch.max_seq_len) <= SCRATCH_BYTES
    hidden, residual = synth.draw_activations(wl.model, T, wl.index, DEV)
    pos, bt, sl = device_batch(batch, DEV)
    qsl = device_qsl(batch, DEV)
    kp, vp = synth.build_kv_pool(wl, batch, 0, DEV)
    kp2, vp2 = kp.clone(), vp.clone()
    ho, ro = layer.forward(hidden, residual, pos, kp, vp, bt, sl, batch.max_seq_len, query_start_loc=qsl)
    ho2 = torch.full_like(hidden, 3.0)
    ro2 = torch.full_like(hidden, 3.0)
    layer.forward_noalloc(hidden, residual, pos, kp2, vp2, bt, sl, batch.max_seq_len, ho2, ro2, query_start_loc=qsl)
    torch.cuda.synchronize()
    for a, b in ((ho, ho2), (ro, ro2), (kp, kp2), (vp, vp2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noalloc_matches_forward_two_calls_then_rejects_oversize():
    w = synth.draw_weights(MID, 80, 0, DEV)
    layer = lda.Layer(MID.config_dict(), w)
    try:
        # a decode batch with long contexts (key partitions, split-K partials in the scratch) ...
        _both(layer, synth.Workload(80, "noalloc_decode_b48", MID, 48, 1, (100, 9000)))
        # ... then a smaller mixed batch: prefill chunks and decode rows
        mix = ((1, 300), (20, 40), (1, 7))
        _both(layer, synth.Workload(81, "noalloc_mixed_3seq", MID, len(mix), 0, mix=mix))
        # a prefill whose workspace exceeds the scratch: rejected, nothing written
        wl = synth.Workload(82, "noalloc_prefill_4x2048", MID, 4, 2048, 0)
        batch = synth.build_batch(wl)
        T, B = batch.num_tokens, batch.num_seqs
        assert layer.workspace_bytes(T, B, batch.max_seq_len) > SCRATCH_BYTES
        hidden, residual = synth.draw_activations(MID, T, wl.index, DEV)
        pos, bt, sl = device_batch(batch, DEV)
        kp, vp = synth.build_kv_pool(wl, batch, 0, DEV)
        kp0, vp0 = kp.clone(), vp.clone()
        ho = torch.full_like(hidden, 5.0)
        ro = torch.full_like(hidden, 5.0)
        with pytest.raises(lda.LlamaError, match="no-allocation forward holds at most") as ei:
            layer.forward_noalloc(hidden, residual, pos, kp, vp, bt, sl, batch.max_seq_len, ho, ro)
        assert ei.value.status == lda.Status.INVALID_ARGUMENT
        torch.cuda.synchronize()
        assert bool((ho == 5.0).all()) and bool((ro == 5.0).all())
        assert torch.equal(kp.view(torch.int16), kp0.view(torch.int16))
        assert torch.equal(vp.view(torch.int16), vp0.view(torch.int16))
    finally:
        layer.close()
