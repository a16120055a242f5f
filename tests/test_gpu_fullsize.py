"""GPU parity at the full 70B-shape workloads, in the launch configuration the
benchmark times.  The oracle runs every row where it can (decode) and sampled
rows elsewhere (prefill: rows spread over each sequence, including the first
and the last position; the oracle still computes K/V for every token those
rows attend to).  Every new K/V slot of the batch is compared, and the cache
placement is checked bit-exact over the whole pool."""
import numpy as np
import pytest
import torch

import llama_decoder_layer_amd as lda
import oracle
import synth
from tests.parity import compare, device_batch, device_qsl, np64, oracle_seqs, oracle_weights, run_oracle
from tests.test_gpu_layer import _check_kv, _check_placement

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"


def _forward(wl, batch, layer_idx, h, r):
    model = wl.model
    w = synth.draw_weights(model, wl.index, layer_idx, DEV)
    kp, vp = synth.build_kv_pool(wl, batch, layer_idx, DEV)
    kp0, vp0 = kp.clone(), vp.clone()
    layer = lda.Layer(model.config_dict(), w)
    pos, bt, sl = device_batch(batch, DEV)
    ho, ro = layer.forward(h, r, pos, kp, vp, bt, sl, batch.max_seq_len, query_start_loc=device_qsl(batch, DEV))
    torch.cuda.synchronize()
    layer.close()
    return w, kp0, vp0, kp, vp, ho, ro


def _sample_rows(batch, per_seq):
    rows = []
    for b in range(batch.num_seqs):
        q, s = batch.new_rows(b), batch.row_start(b)
        picks = sorted({0, 1, 15, 16, 17, q // 3, q // 2, q - 17, q - 2, q - 1} | set(per_seq))
        rows += [s + i for i in picks if 0 <= i < q]
    return rows


def _check_prefill(name, extra=()):
    wl = synth.WORKLOADS[name]
    batch = synth.build_batch(wl)
    print("case", name, "T", batch.num_tokens, flush=True)
    hidden, residual = synth.draw_activations(wl.model, batch.num_tokens, wl.index, DEV)
    w, kp0, vp0, kp, vp, ho, ro = _forward(wl, batch, 0, hidden, residual)
    want = _sample_rows(batch, extra)
    seqs = oracle_seqs(wl.model, batch, kp0, vp0)
    wn = oracle_weights(w)
    exact, rounded = run_oracle(wl.model, wn, hidden, residual, batch, seqs, want=want)
    idx = torch.tensor(want, device=DEV)
    s1 = compare("hidden_out", np64(ho[idx]), exact["hidden_out"], rounded["hidden_out"])
    s2 = compare("residual_out", np64(ro[idx]), exact["residual_out"], rounded["residual_out"])
    print("rows", len(want), "hidden_out", s1, "residual_out", s2, flush=True)
    _check_kv(wl.model, batch, kp0, vp0, kp, vp, exact, rounded)


def test_c1_decode_b32_ctx2048_all_rows():
    wl = synth.WORKLOADS["llama70b_decode_b32_ctx2048"]
    batch = synth.build_batch(wl)
    hidden, residual = synth.draw_activations(wl.model, batch.num_tokens, wl.index, DEV)
    w, kp0, vp0, kp, vp, ho, ro = _forward(wl, batch, 0, hidden, residual)
    seqs = oracle_seqs(wl.model, batch, kp0, vp0)
    exact, rounded = run_oracle(wl.model, oracle_weights(w), hidden, residual, batch, seqs)
    s1 = compare("hidden_out", np64(ho), exact["hidden_out"], rounded["hidden_out"])
    s2 = compare("residual_out", np64(ro), exact["residual_out"], rounded["residual_out"])
    print("hidden_out", s1, "residual_out", s2, flush=True)
    _check_kv(wl.model, batch, kp0, vp0, kp, vp, exact, rounded)


@pytest.mark.timeout(600)
def test_c2_prefill_4x2048_sampled_rows():
    _check_prefill("llama70b_prefill_4x2048", extra=(511, 512, 1023, 1024))


@pytest.mark.timeout(900)
def test_c3_prefill_1x32768_sampled_rows():
    # positions past the llama3 original context (8192) included
    _check_prefill("llama70b_prefill_1x32768", extra=(4095, 8191, 8192, 8193, 16384, 24575, 30000))


@pytest.mark.timeout(900)
def test_c4_ragged_decode_4layer_sampled_sequences():
    wl = synth.WORKLOADS["llama70b_ragged_decode_b64_4layer"]
    batch = synth.build_batch(wl)
    lens = batch.ctx_lens
    # the shortest, the longest and a spread of others
    order = sorted(range(batch.num_seqs), key=lambda b: lens[b])
    pick = sorted({order[0], order[1], order[-1], order[-2], order[len(order) // 2], 0, 13, 41})
    print("ctx of sampled sequences", [lens[b] for b in pick], flush=True)
    hidden, residual = synth.draw_activations(wl.model, batch.num_tokens, wl.index, DEV)
    h, r = hidden, residual
    per_layer = []
    for l in range(wl.layers):
        w, kp0, vp0, kp, vp, ho, ro = _forward(wl, batch, l, h, r)
        _check_placement(wl.model, batch, kp0, vp0, kp, vp)
        seqs = oracle_seqs(wl.model, batch, kp0, vp0, seq_ids=pick)
        knew, vnew = [], []
        for b in pick:
            p = lens[b]
            blk = int(batch.block_table[b, p // 16])
            knew.append(np64(kp[blk, :, p % 16, :]))
            vnew.append(np64(vp[blk, :, :, p % 16]))
        del kp0, vp0, kp, vp
        per_layer.append((w, seqs, ho[pick].clone(), ro[pick].clone(), knew, vnew))
        h, r = ho, ro
    cfg = wl.model.config_dict()
    pos = batch.positions.numpy().astype(np.int64)
    he, re_ = np64(hidden), np64(residual)
    hr, rr = he.copy(), re_.copy()
    for l, (w, seqs, ho, ro, knew, vnew) in enumerate(per_layer):
        wn = oracle_weights(w)
        ex = oracle.decoder_layer(cfg, wn, he, re_, pos, seqs, want=pick)
        rd = oracle.decoder_layer(cfg, wn, hr, rr, pos, seqs, rnd=oracle.bf16_round, want=pick)
        s1 = compare("hidden_out[%d]" % l, np64(ho), ex["hidden_out"], rd["hidden_out"], depth=l + 1)
        s2 = compare("residual_out[%d]" % l, np64(ro), ex["residual_out"], rd["residual_out"], depth=l + 1)
        print("layer", l, "hidden_out", s1, "residual_out", s2, flush=True)
        # new K/V of the sampled sequences
        compare("k_cache[%d]" % l, np.stack(knew), np.stack([k[0] for k in ex["k_new"]]),
                np.stack([k[0] for k in rd["k_new"]]), depth=l + 1)
        compare("v_cache[%d]" % l, np.stack(vnew), np.stack([v[0] for v in ex["v_new"]]),
                np.stack([v[0] for v in rd["v_new"]]), depth=l + 1)
        he, re_ = he.copy(), re_.copy()
        he[pick], re_[pick] = ex["hidden_out"], ex["residual_out"]
        hr, rr = hr.copy(), rr.copy()
        hr[pick], rr[pick] = oracle.bf16_round(rd["hidden_out"]), oracle.bf16_round(rd["residual_out"])
        del wn


@pytest.mark.timeout(600)
def test_mixed_chunk512_decode32_sampled_rows():
    # one call with 32 decode rows (context 2048) and a 512-row prefill chunk
    # on a 4096-token context: every decode row, sampled chunk rows
    _check_prefill("llama70b_mixed_chunk512_decode32", extra=(255, 256, 511))


def test_qwen3moe_decode_b32_ctx2048_all_rows():
    # the Qwen3-30B-A3B layer: 128 experts, top-8, q/k norm
    from tests.test_gpu_moe import run_moe_layer
    run_moe_layer(synth.WORKLOADS["qwen3moe_decode_b32_ctx2048"])


@pytest.mark.timeout(600)
def test_qwen3moe_prefill_4x2048_sampled_rows():
    from tests.test_gpu_moe import run_moe_layer
    wl = synth.WORKLOADS["qwen3moe_prefill_4x2048"]
    batch = synth.build_batch(wl)
    # each sequence's last row is sampled, so the oracle forms every new K/V
    run_moe_layer(wl, want=_sample_rows(batch, (511, 512, 1023, 1024)), check_kv=True)


def test_tp8_shard_decode_b32_ctx2048_all_rows():
    # one GPU's TP = 8 share of the 70B layer: qkv N = 1280, o_proj K = 1024,
    # gate_up N = 2 x 3584, down K = 3584, attention 8 query heads on 1 KV head
    wl = synth.WORKLOADS["llama70b_tp8shard_decode_b32_ctx2048"]
    batch = synth.build_batch(wl)
    hidden, residual = synth.draw_activations(wl.model, batch.num_tokens, wl.index, DEV)
    w, kp0, vp0, kp, vp, ho, ro = _forward(wl, batch, 0, hidden, residual)
    seqs = oracle_seqs(wl.model, batch, kp0, vp0)
    exact, rounded = run_oracle(wl.model, oracle_weights(w), hidden, residual, batch, seqs)
    s1 = compare("hidden_out", np64(ho), exact["hidden_out"], rounded["hidden_out"])
    s2 = compare("residual_out", np64(ro), exact["residual_out"], rounded["residual_out"])
    print("hidden_out", s1, "residual_out", s2, flush=True)
    _check_kv(wl.model, batch, kp0, vp0, kp, vp, exact, rounded)


@pytest.mark.timeout(600)
def test_tp8_shard_prefill_4x2048_sampled_rows():
    _check_prefill("llama70b_tp8shard_prefill_4x2048", extra=(511, 512, 1023, 1024))
