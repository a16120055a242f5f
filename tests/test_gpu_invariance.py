"""Invariances of the paged forward, checked on the library itself (the
oracle has its own pins for the same properties):

* moving every cache block to another physical id -- block table and pool
  contents permuted together -- changes no output bit, and every cache bit
  ends up at the moved slot;
* a sequence's outputs and its new K/V slots do not depend on its
  batch-mates' values, nor on its index in the batch (same batch shape, so
  the same launch plan): bitwise;
* a prefill of S tokens, and a prefill of S - 1 tokens followed by a decode
  of the last one, write the same cache bits for the first S - 1 positions
  and agree with the oracle on the last token.

Pages: "模型库与算子层 — 代码走读", "Attention 层" (the new k and v are written
into the paged cache before attention reads it through the block table);
"vLLM Llama 代码解析" §2.1 (one forward over a batch of sequences)."""
import dataclasses

import numpy as np
import pytest
import torch

import llama_decoder_layer_amd as lda
import synth
from tests.parity import compare, np64, oracle_seqs, oracle_weights, run_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"

MID = synth.ModelShape(1024, 8, 2, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")
MID8 = synth.ModelShape(1024, 8, 1, 128, 2816, 1e-5, 500000.0, synth.LLAMA3_SCALING, 131072, "bf16")


def _forward(model, w, batch, hidden, residual, kp, vp):
    """One forward on copies of the pools; returns (hidden_out, residual_out,
    k_pool, v_pool) after the call."""
    kp, vp = kp.clone(), vp.clone()
    pos, bt, sl = batch.positions.to(DEV), batch.block_table.to(DEV), batch.seq_lens.to(DEV)
    qsl = batch.query_start_loc
    qsl = None if qsl is None else qsl.to(DEV)
    layer = lda.Layer(model.config_dict(), w)
    ws = layer.alloc_workspace(batch.num_tokens, batch.num_seqs, batch.max_seq_len)
    ho, ro = layer.forward(hidden, residual, pos, kp, vp, bt, sl, batch.max_seq_len, workspace=ws,
                           query_start_loc=qsl)
    torch.cuda.synchronize()
    layer.close()
    return ho, ro, kp, vp


def _bits(t):
    return t.contiguous().view(torch.int16)


def _same(a, b):
    return torch.equal(_bits(a), _bits(b))


CASES = {
    # decode rows with key partitions (and the combine), block edges, an empty context
    "decode": lambda: (synth.Workload(60, "inv_decode_b6", MID, 6, 1, 0), [0, 15, 16, 300, 1000, 3000]),
    # prefill chunks on cached contexts (8 query heads per KV head)
    "prefill_ctx": lambda: (synth.Workload(61, "inv_prefill_3x37_ctx", MID8, 3, 37, 0), [5, 300, 64]),
    # decode rows, prefill chunks and a fresh prefill in one call
    "mixed": lambda: (synth.Workload(62, "inv_mixed_5seq", MID, 5, 0,
                                     mix=((1, 300), (37, 50), (64, 0), (1, 2000), (20, 777))), None),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_block_relocation_changes_no_bit(case):
    wl, ctx = CASES[case]()
    model = wl.model
    batch = synth.build_batch(wl, ctx)
    print("case", case, "ctx", batch.ctx_lens, "T", batch.num_tokens, flush=True)
    hidden, residual = synth.draw_activations(model, batch.num_tokens, wl.index, DEV)
    w = synth.draw_weights(model, wl.index, 0, DEV)
    kp, vp = synth.build_kv_pool(wl, batch, 0, DEV)
    # block i moves to id sigma[i]: the table's entries and the pool's blocks together
    g = torch.Generator().manual_seed(1000 + wl.index)
    sigma = torch.randperm(batch.num_blocks, generator=g)
    table = batch.block_table.clone()
    live = table >= 0
    table[live] = sigma[table[live].long()].to(torch.int32)
    moved = dataclasses.replace(batch, block_table=table)
    sd = sigma.to(DEV)
    kp_m, vp_m = torch.empty_like(kp), torch.empty_like(vp)
    kp_m[sd] = kp
    vp_m[sd] = vp

    ho, ro, kp1, vp1 = _forward(model, w, batch, hidden, residual, kp, vp)
    ho_m, ro_m, kp1_m, vp1_m = _forward(model, w, moved, hidden, residual, kp_m, vp_m)
    assert _same(ho, ho_m) and _same(ro, ro_m), "outputs depend on where the blocks sit"
    assert _same(kp1_m[sd], kp1) and _same(vp1_m[sd], vp1), "cache bits not at the moved slots"


def _permuted_batch(batch, order):
    """The same sequences in batch order `order` (new index i holds old
    sequence order[i]), with their rows, positions and block-table rows."""
    rows = [r for b in order for r in batch.rows(b)]
    q_lens = None if batch.q_lens is None else [batch.q_lens[b] for b in order]
    nb = dataclasses.replace(batch, ctx_lens=[batch.ctx_lens[b] for b in order],
                             seq_lens=batch.seq_lens[order].clone(), positions=batch.positions[rows].clone(),
                             block_table=batch.block_table[order].clone(), q_lens=q_lens)
    return nb, rows


@pytest.mark.parametrize("case", ["decode", "prefill_ctx"])
def test_sequence_outputs_independent_of_batch_mates_and_order(case):
    if case == "decode":
        wl = synth.Workload(63, "inv_mates_decode_b8", MID, 8, 1, 0)
        ctx = [700, 50, 1500, 3, 900, 2047, 64, 333]
    else:
        wl = synth.Workload(64, "inv_mates_prefill_4x33", MID8, 4, 33, 0)
        ctx = [100, 0, 257, 16]
    target = 2
    model = wl.model
    batch = synth.build_batch(wl, ctx)
    print("case", case, "ctx", batch.ctx_lens, "T", batch.num_tokens, flush=True)
    T = batch.num_tokens
    hidden, residual = synth.draw_activations(model, T, wl.index, DEV)
    w = synth.draw_weights(model, wl.index, 0, DEV)
    kp, vp = synth.build_kv_pool(wl, batch, 0, DEV)
    ho, ro, kp1, vp1 = _forward(model, w, batch, hidden, residual, kp, vp)
    trows = list(batch.rows(target))
    tblocks = batch.block_table[target]
    tblocks = tblocks[tblocks >= 0].long().to(DEV)

    # other values for every other sequence: rows and cached contexts
    other = dataclasses.replace(wl, index=wl.index + 100)
    h2, r2 = synth.draw_activations(model, T, other.index, DEV)
    h2[trows], r2[trows] = hidden[trows], residual[trows]
    kp2, vp2 = synth.build_kv_pool(other, batch, 0, DEV)
    kp2[tblocks], vp2[tblocks] = kp[tblocks], vp[tblocks]
    ho2, ro2, kp3, vp3 = _forward(model, w, batch, h2, r2, kp2, vp2)
    assert _same(ho2[trows], ho[trows]) and _same(ro2[trows], ro[trows]), "outputs depend on batch-mates"
    assert _same(kp3[tblocks], kp1[tblocks]) and _same(vp3[tblocks], vp1[tblocks])

    # the same sequences in another order (the target moves from index 2 to 5)
    order = [3, 7, 0, 6, 1, target, 4, 5]
    order = order[:batch.num_seqs] if batch.num_seqs == 8 else [3, 0, 1, target][:batch.num_seqs]
    assert sorted(order) == list(range(batch.num_seqs))
    pb, rows = _permuted_batch(batch, order)
    ho4, ro4, kp4, vp4 = _forward(model, w, pb, hidden[rows].clone(), residual[rows].clone(), kp, vp)
    new_t = order.index(target)
    prow = list(pb.rows(new_t))
    assert _same(ho4[prow], ho[trows]) and _same(ro4[prow], ro[trows]), "outputs depend on the batch index"
    assert _same(kp4, kp1) and _same(vp4, vp1), "cache differs with the batch order"


def test_prefill_then_decode_matches_prefill():
    S = 200
    wl = synth.Workload(65, "inv_prefill_2x200", MID, 2, S, 0)
    model = wl.model
    full = synth.build_batch(wl, [0, 0])
    hidden, residual = synth.draw_activations(model, full.num_tokens, wl.index, DEV)
    w = synth.draw_weights(model, wl.index, 0, DEV)
    kp, vp = synth.build_kv_pool(wl, full, 0, DEV)  # no cached context: sentinel only
    B = full.num_seqs
    head = [b * S + i for b in range(B) for i in range(S - 1)]
    last = [b * S + S - 1 for b in range(B)]
    # the same sequences and blocks: S - 1 rows first, then one decode row
    pre = dataclasses.replace(full, q_len=S - 1, seq_lens=torch.full((B,), S - 1, dtype=torch.int32),
                              positions=full.positions[head].clone())
    dec = dataclasses.replace(full, q_len=1, ctx_lens=[S - 1] * B, positions=full.positions[last].clone())

    ho, ro, kp1, vp1 = _forward(model, w, full, hidden, residual, kp, vp)
    _, _, kpp, vpp = _forward(model, w, pre, hidden[head].clone(), residual[head].clone(), kp, vp)
    hd, rd, kpd, vpd = _forward(model, w, dec, hidden[last].clone(), residual[last].clone(), kpp, vpp)

    # the first S - 1 positions: the same projection plan and RoPE, bit for bit
    for b in range(B):
        for plane, a, c in (("k", kp1, kpd), ("v", vp1, vpd)):
            x = synth.gather_context(a, full, b, S - 1, plane)
            y = synth.gather_context(c, full, b, S - 1, plane)
            assert _same(x, y), (plane, b)
    # the last token: both paths against the oracle under the parity tolerance
    seqs = oracle_seqs(model, full, kp, vp)
    wn = oracle_weights(w)
    exact, rounded = run_oracle(model, wn, hidden, residual, full, seqs)
    for name, got in (("prefill", ho[last]), ("prefill then decode", hd)):
        st = compare("hidden_out[last] " + name, np64(got), exact["hidden_out"][last], rounded["hidden_out"][last])
        print(name, st, flush=True)
    compare("residual_out[last] prefill then decode", np64(rd), exact["residual_out"][last],
            rounded["residual_out"][last])
    for plane, pool_full, pool_dec, key in (("k", kp1, kpd, "k_new"), ("v", vp1, vpd, "v_new")):
        for b in range(B):
            ref, ref_r = exact[key][b][S - 1:S], rounded[key][b][S - 1:S]
            for name, pool in (("prefill", pool_full), ("decode", pool_dec)):
                got = np64(synth.gather_context(pool, full, b, S, plane)[S - 1:S])
                compare("%s_cache[%d] last slot %s" % (plane, b, name), got, ref, ref_r)
    assert np.all(np.isfinite(np64(hd)))
